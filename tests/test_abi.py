"""The C ABI library loads, exports what include/rmx.h declares, and rejects bad
arguments on the host before touching a GPU (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

import rankmixer_block_forward_amd as rmx
from rankmixer_block_forward_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "rmx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rmx_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = rmx.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.rmx_abi_version() == 6


def test_status_strings_and_kernel_names():
    lib = rmx.load_library()
    for s in range(5):
        assert lib.rmx_status_string(s)
    assert lib.rmx_status_string(99) == b"unknown status"
    names = [lib.rmx_kernel_name(i) for i in range(binding.KERNEL_COUNT)]
    assert len(set(names)) == binding.KERNEL_COUNT and lib.rmx_kernel_name(-1) == b"unknown"


def _create(**kw):
    lib = rmx.load_library()
    base = dict(T=4, D=8, k=2, L=1, dtype=binding.RMX_FP32, ln_eps=1e-5, max_batch=8, moe_experts=0, moe_hidden=0,
                routing=binding.RMX_ROUTING_MIX)
    base.update(kw)
    cfg = binding.rmx_config(**base)
    h = ctypes.c_void_p(1234)
    st = lib.rmx_create(ctypes.byref(cfg), ctypes.byref(h))
    return st, h, lib.rmx_last_error(None).decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(D=9), binding.RMX_ERR_INVALID_ARG, "not divisible"),
    (dict(T=0), binding.RMX_ERR_INVALID_ARG, ">= 1"),
    (dict(L=0), binding.RMX_ERR_INVALID_ARG, ">= 1"),
    (dict(dtype=7), binding.RMX_ERR_INVALID_ARG, "dtype"),
    (dict(ln_eps=0.0), binding.RMX_ERR_INVALID_ARG, "ln_eps"),
    (dict(max_batch=-1), binding.RMX_ERR_INVALID_ARG, "max_batch"),
    (dict(dtype=binding.RMX_BF16, T=4, D=8), binding.RMX_ERR_UNSUPPORTED, "D/T"),
    (dict(T=32, D=1536, dtype=binding.RMX_FP32), binding.RMX_ERR_UNSUPPORTED, "LDS"),
    (dict(D=8192, T=1), binding.RMX_ERR_UNSUPPORTED, "row kernel limit"),
    (dict(D=520, T=130), binding.RMX_ERR_UNSUPPORTED, "row kernel limit"),
    (dict(routing=7), binding.RMX_ERR_INVALID_ARG, "routing"),
    (dict(routing=binding.RMX_ROUTING_ATTENTION, T=65, D=130), binding.RMX_ERR_UNSUPPORTED, "attention"),
])
def test_create_rejects_bad_configs_on_the_host(kw, status, text):
    st, h, msg = _create(**kw)
    assert st == status, msg
    assert h.value is None
    assert text in msg


def test_null_arguments():
    lib = rmx.load_library()
    assert lib.rmx_destroy(None) == binding.RMX_OK
    assert lib.rmx_block_forward(None, None, 1, None, 1, 1, None, None) == binding.RMX_ERR_INVALID_ARG
    assert lib.rmx_create(None, None) == binding.RMX_ERR_INVALID_ARG
    assert lib.rmx_profile_enable(None, 1) == binding.RMX_ERR_INVALID_ARG
    assert lib.rmx_token_mix(None, None, 1, 3, 8, 0, None) == binding.RMX_ERR_INVALID_ARG
    assert "divisible" in lib.rmx_last_error(None).decode()
    assert lib.rmx_token_mix(None, None, 0, 4, 8, 0, None) == binding.RMX_OK  # B = 0: nothing to do


def test_tokenize_host_side_rejections():
    """Argument errors of rmx_tokenize are caught on the host before any GPU work."""
    lib = rmx.load_library()
    assert lib.rmx_tokenize(None, None, None, None, 1, 0, 4, 8, 0, None) == binding.RMX_ERR_INVALID_ARG
    assert ">= 1" in lib.rmx_last_error(None).decode()
    assert lib.rmx_tokenize(None, None, None, None, 1, 2, 4, 8, 7, None) == binding.RMX_ERR_INVALID_ARG
    assert "dtype" in lib.rmx_last_error(None).decode()
    assert lib.rmx_tokenize(None, None, None, None, 0, 2, 4, 8, 1, None) == binding.RMX_OK  # B = 0
    assert lib.rmx_tokenize(None, None, None, None, -1, 2, 4, 8, 1, None) == binding.RMX_ERR_INVALID_ARG


def test_packed_weights_host_side():
    lib = rmx.load_library()
    assert lib.rmx_packed_weights_bytes(None) == 0
    assert lib.rmx_pack_weights(None, None, 1, None, 0, None) == binding.RMX_ERR_INVALID_ARG


def test_training_entry_points_host_side():
    """Without a handle, the training entry points reject their arguments on the host."""
    lib = rmx.load_library()
    assert lib.rmx_saved_bytes(None, 8) == 0
    assert lib.rmx_block_forward_train(None, None, 1, None, 1, 1, None, None, 0, None) == binding.RMX_ERR_INVALID_ARG
    assert lib.rmx_block_backward(None, None, 1, None, 1, 1, None, 0, None, None, None, None) == \
        binding.RMX_ERR_INVALID_ARG
    assert "handle" in lib.rmx_last_error(None).decode()


def test_grads_struct_matches_header():
    """rmx_grads in the binding lists the header's fields in order."""
    src = open(os.path.join(ROOT, "include", "rmx.h")).read()
    body = re.search(r"typedef struct \{([^}]*)\} rmx_grads;", src).group(1)
    fields = re.findall(r"float\*\s+(\w+);", body)
    assert fields == [f for f, _ in binding.rmx_grads._fields_]


def test_mxfp8_host_side():
    lib = rmx.load_library()
    assert lib.rmx_packed_weights_mxfp8_bytes(None) == 0
    assert lib.rmx_pack_weights_mxfp8(None, None, 1, None, 0, None) == binding.RMX_ERR_INVALID_ARG


def test_weights_struct_matches_header():
    src = open(os.path.join(ROOT, "include", "rmx.h")).read()
    body = re.search(r"typedef struct \{([^}]*)\} rmx_weights;", src).group(1)
    fields = re.findall(r"const void\*\s+(\w+);", body)
    assert fields == list(binding.WEIGHT_NAMES)


def test_config_struct_matches_header():
    src = open(os.path.join(ROOT, "include", "rmx.h")).read()
    body = re.search(r"typedef struct \{([^}]*)\} rmx_config;", src).group(1)
    fields = re.findall(r"(?:int32_t|int64_t|float)\s+(\w+);", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert fields == [f for f, _ in binding.rmx_config._fields_]
