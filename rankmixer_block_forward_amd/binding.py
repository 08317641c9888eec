"""Python binding of librmx.so (include/rmx.h): argument marshalling only.

Every step of the forward pass runs in the library's HIP kernels; this module only
checks that tensors are on the GPU with the right dtype and layout and passes their
device pointers and the current HIP stream.  PyTorch provides the device memory and
streams.  There is no fallback: if librmx.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librmx.so")

RMX_OK, RMX_ERR_INVALID_ARG, RMX_ERR_UNSUPPORTED, RMX_ERR_OUT_OF_MEMORY, RMX_ERR_HIP = range(5)
RMX_FP32, RMX_BF16 = 0, 1
RMX_ROUTING_MIX, RMX_ROUTING_ATTENTION = 0, 1
KERNEL_COUNT = 16

# Every symbol include/rmx.h declares.
EXPORTS = (
    "rmx_create", "rmx_destroy", "rmx_block_forward", "rmx_block_forward_ex", "rmx_block_forward_moe_lists",
    "rmx_token_mix",
    "rmx_tokenize", "rmx_packed_weights_bytes", "rmx_pack_weights",
    "rmx_packed_weights_mxfp8_bytes", "rmx_pack_weights_mxfp8",
    "rmx_saved_bytes", "rmx_block_forward_train", "rmx_block_backward",
    "rmx_profile_enable", "rmx_profile_read", "rmx_profile_reset", "rmx_kernel_name",
    "rmx_status_string", "rmx_last_error", "rmx_abi_version", "rmx_block_forward_noalloc",
)


class RmxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"rmx status {status}: {message}")
        self.status = status


class rmx_config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("k", ctypes.c_int32),
                ("L", ctypes.c_int32), ("dtype", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("max_batch", ctypes.c_int64), ("moe_experts", ctypes.c_int32),
                ("moe_hidden", ctypes.c_int32), ("routing", ctypes.c_int32)]


WEIGHT_NAMES = ("W1", "b1", "W2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b",
                "Wg", "We1", "be1", "We2", "be2", "packed", "packed_mxfp8", "Wq", "Wk", "Wv")


class rmx_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


GRAD_NAMES = ("W1", "b1", "W2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")


MOE_LIST_NAMES = ("group_start", "rows", "row_gate", "pos", "tile_start")


class rmx_moe_lists(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in MOE_LIST_NAMES]


class rmx_grads(ctypes.Structure):
    _fields_ = [("d" + n, ctypes.c_void_p) for n in GRAD_NAMES]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads librmx.so once; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run python -m rankmixer_block_forward_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.rmx_create.argtypes = [ctypes.POINTER(rmx_config), ctypes.POINTER(vp)]
    lib.rmx_destroy.argtypes = [vp]
    lib.rmx_block_forward.argtypes = [vp, vp, i64, ctypes.POINTER(rmx_weights), i32, i32, vp, vp]
    lib.rmx_block_forward_ex.argtypes = [vp, vp, i64, ctypes.POINTER(rmx_weights), i32, i32, vp,
                                         vp, vp, vp]
    lib.rmx_block_forward_moe_lists.argtypes = [vp, vp, i64, ctypes.POINTER(rmx_weights), i32, i32, vp, vp, vp,
                                                ctypes.POINTER(rmx_moe_lists), vp]
    lib.rmx_block_forward_noalloc.argtypes = [ctypes.POINTER(rmx_config), vp, i64, ctypes.POINTER(rmx_weights),
                                              vp, vp]
    lib.rmx_token_mix.argtypes = [vp, vp, i64, i32, i32, i32, vp]
    lib.rmx_tokenize.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, vp]
    lib.rmx_packed_weights_bytes.argtypes = [vp]
    lib.rmx_packed_weights_bytes.restype = ctypes.c_size_t
    lib.rmx_pack_weights.argtypes = [vp, ctypes.POINTER(rmx_weights), i32, vp, ctypes.c_size_t, vp]
    lib.rmx_packed_weights_mxfp8_bytes.argtypes = [vp]
    lib.rmx_packed_weights_mxfp8_bytes.restype = ctypes.c_size_t
    lib.rmx_pack_weights_mxfp8.argtypes = [vp, ctypes.POINTER(rmx_weights), i32, vp, ctypes.c_size_t, vp]
    lib.rmx_saved_bytes.argtypes = [vp, i64]
    lib.rmx_saved_bytes.restype = ctypes.c_size_t
    lib.rmx_block_forward_train.argtypes = [vp, vp, i64, ctypes.POINTER(rmx_weights), i32, i32, vp, vp,
                                            ctypes.c_size_t, vp]
    lib.rmx_block_backward.argtypes = [vp, vp, i64, ctypes.POINTER(rmx_weights), i32, i32, vp, ctypes.c_size_t,
                                       vp, vp, ctypes.POINTER(rmx_grads), vp]
    lib.rmx_profile_enable.argtypes = [vp, i32]
    lib.rmx_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64),
                                     ctypes.POINTER(i64)]
    lib.rmx_profile_reset.argtypes = [vp]
    lib.rmx_kernel_name.argtypes = [i32]
    lib.rmx_kernel_name.restype = ctypes.c_char_p
    lib.rmx_status_string.argtypes = [ctypes.c_int]
    lib.rmx_status_string.restype = ctypes.c_char_p
    lib.rmx_last_error.argtypes = [vp]
    lib.rmx_last_error.restype = ctypes.c_char_p
    lib.rmx_abi_version.restype = i32
    for name in EXPORTS:
        if name not in ("rmx_kernel_name", "rmx_status_string", "rmx_last_error", "rmx_abi_version",
                        "rmx_packed_weights_bytes", "rmx_saved_bytes", "rmx_packed_weights_mxfp8_bytes"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, handle=None):
    if status != RMX_OK:
        lib = load_library()
        msg = lib.rmx_last_error(handle).decode()
        raise RmxError(status, f"{lib.rmx_status_string(status).decode()}: {msg}")


def _dtype_code(dtype) -> int:
    import torch
    if dtype in ("bf16", torch.bfloat16, RMX_BF16):
        return RMX_BF16
    if dtype in ("fp32", torch.float32, RMX_FP32):
        return RMX_FP32
    raise ValueError(f"unsupported dtype {dtype}")


def _torch_dtype(code: int):
    import torch
    return torch.bfloat16 if code == RMX_BF16 else torch.float32


def _ptr(t, name, dtype=None, shape=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _weights_struct(w: dict, dtype) -> rmx_weights:
    import torch
    s = rmx_weights()
    for n in WEIGHT_NAMES:
        t = w.get(n)
        setattr(s, n, _ptr(t, n, torch.uint8 if n == "packed_mxfp8" else dtype))
    return s


def forward_noalloc(X, weights: dict, T: int, D: int, k: int, L: int, dtype="bf16", ln_eps: float = 1e-5,
                    out=None, stream=None):
    """rmx_block_forward_noalloc: the dense forward with the library's fixed device
    workspace (no handle, no device allocation by the library).  `out` may be given so
    that the call allocates nothing on the Python side either."""
    import torch
    lib = load_library()
    code = _dtype_code(dtype)
    B = X.shape[0]
    _ptr(X, "X", _torch_dtype(code), (B, T, D))
    if out is None:
        out = torch.empty((B, D), dtype=torch.float32, device=X.device)
    _ptr(out, "out", torch.float32, (B, D))
    cfg = rmx_config(T, D, k, L, code, ln_eps, B, 0, 0, RMX_ROUTING_MIX)
    ws = _weights_struct(weights, _torch_dtype(code))
    _check(lib.rmx_block_forward_noalloc(ctypes.byref(cfg), _ptr(X, "X"), B, ctypes.byref(ws), _ptr(out, "out"),
                                         _stream(stream)))
    return out


class Handle:
    """One rmx_handle: a model configuration and its workspace on the current device."""

    def __init__(self, T: int, D: int, k: int, L: int, dtype="bf16", ln_eps: float = 1e-5,
                 max_batch: int = 2048, moe_experts: int = 0, moe_hidden: int = 0, routing: str = "mix"):
        self._lib = load_library()
        if routing not in ("mix", "attention"):
            raise ValueError(f"unknown routing {routing!r}")
        code = RMX_ROUTING_ATTENTION if routing == "attention" else RMX_ROUTING_MIX
        self.cfg = rmx_config(T, D, k, L, _dtype_code(dtype), ln_eps, max_batch, moe_experts, moe_hidden, code)
        self.dtype = _torch_dtype(self.cfg.dtype)
        h = ctypes.c_void_p()
        _check(self._lib.rmx_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h

    @classmethod
    def for_config(cls, cfg, max_batch: int | None = None) -> "Handle":
        """Handle for a synth.Config workload."""
        return cls(cfg.T, cfg.D, cfg.k, cfg.L, cfg.dtype, cfg.eps,
                   cfg.B if max_batch is None else max_batch, cfg.E, cfg.moe_hidden, cfg.routing)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.rmx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _weights(self, w: dict) -> rmx_weights:
        return _weights_struct(w, self.dtype)

    def packed_weights_bytes(self) -> int:
        """Bytes of the prepared copy of W1 and W2 (0 when this handle has no such path)."""
        return int(self._lib.rmx_packed_weights_bytes(self._h))

    def pack_weights(self, weights: dict, stream=None):
        """W1 and W2 (We1 and We2 for a Sparse-MoE handle) of all blocks prepared for the
        matrix cores (rmx_pack_weights): a device tensor to pass as weights["packed"]; the
        forward then reads those weights from it."""
        import torch
        nbytes = self.packed_weights_bytes()
        if nbytes == 0:
            raise RmxError(RMX_ERR_UNSUPPORTED, "this handle has no prepared-weights path")
        packed = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        names = ("We1", "We2") if self.cfg.moe_experts > 0 else ("W1", "W2")
        ws = self._weights({n: weights[n] for n in names})
        _check(self._lib.rmx_pack_weights(self._h, ctypes.byref(ws), self.cfg.L, _ptr(packed, "packed"), nbytes,
                                          _stream(stream)), self._h)
        return packed

    def packed_weights_mxfp8_bytes(self) -> int:
        """Bytes of W1 and W2 in MXFP8 (0 when this handle has no such path)."""
        return int(self._lib.rmx_packed_weights_mxfp8_bytes(self._h))

    def pack_weights_mxfp8(self, weights: dict, stream=None):
        """W1 and W2 of all blocks quantized to MXFP8 (rmx_pack_weights_mxfp8): a device byte
        tensor to pass as weights["packed_mxfp8"]; the forward then runs the MXFP8 variant."""
        import torch
        nbytes = self.packed_weights_mxfp8_bytes()
        if nbytes == 0:
            raise RmxError(RMX_ERR_UNSUPPORTED, "this handle has no MXFP8 path")
        packed = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ws = self._weights({"W1": weights["W1"], "W2": weights["W2"]})
        _check(self._lib.rmx_pack_weights_mxfp8(self._h, ctypes.byref(ws), self.cfg.L, _ptr(packed, "packed"),
                                                nbytes, _stream(stream)), self._h)
        return packed

    def forward(self, X, weights: dict, out=None, xl_out=None, gate_out=None, stream=None,
                L: int | None = None, k: int | None = None):
        """out[B, D] (fp32) = mean-pooled X_L of the L blocks over X[B, T, D]."""
        import torch
        c = self.cfg
        B = X.shape[0]
        _ptr(X, "X", self.dtype, (B, c.T, c.D))
        if out is None:
            out = torch.empty((B, c.D), dtype=torch.float32, device=X.device)
        _ptr(out, "out", torch.float32, (B, c.D))
        _ptr(xl_out, "xl_out", self.dtype, (B, c.T, c.D))
        if gate_out is not None:
            _ptr(gate_out, "gate_out", torch.float32, (c.L, B, c.T, c.moe_experts))
        ws = self._weights(weights)
        st = self._lib.rmx_block_forward_ex(
            self._h, _ptr(X, "X"), B, ctypes.byref(ws), c.L if L is None else L, c.k if k is None else k,
            _ptr(out, "out"), _ptr(xl_out, "xl_out"), _ptr(gate_out, "gate_out"), _stream(stream))
        _check(st, self._h)
        return out

    def forward_moe_lists(self, X, weights: dict, out=None, xl_out=None, gate_out=None, stream=None):
        """Sparse-MoE forward (rmx_block_forward_moe_lists) that also returns the routing lists
        of every block: a dict of device tensors group_start [L, G+1], rows [L, G*B],
        row_gate [L, G*B], pos [L, G, B], tile_start [L, G+1] (G = T*E groups)."""
        import torch
        c = self.cfg
        B = X.shape[0]
        _ptr(X, "X", self.dtype, (B, c.T, c.D))
        if out is None:
            out = torch.empty((B, c.D), dtype=torch.float32, device=X.device)
        _ptr(out, "out", torch.float32, (B, c.D))
        _ptr(xl_out, "xl_out", self.dtype, (B, c.T, c.D))
        if gate_out is not None:
            _ptr(gate_out, "gate_out", torch.float32, (c.L, B, c.T, c.moe_experts))
        G = c.T * c.moe_experts
        i32 = dict(dtype=torch.int32, device=X.device)
        lists = {"group_start": torch.full((c.L, G + 1), -7, **i32),
                 "rows": torch.full((c.L, G * B), -7, **i32),
                 "row_gate": torch.full((c.L, G * B), float("nan"), dtype=torch.float32, device=X.device),
                 "pos": torch.full((c.L, G, B), -7, **i32),
                 "tile_start": torch.full((c.L, G + 1), -7, **i32)}
        ls = rmx_moe_lists(*[lists[n].data_ptr() for n in MOE_LIST_NAMES])
        ws = self._weights(weights)
        st = self._lib.rmx_block_forward_moe_lists(
            self._h, _ptr(X, "X"), B, ctypes.byref(ws), c.L, c.k, _ptr(out, "out"), _ptr(xl_out, "xl_out"),
            _ptr(gate_out, "gate_out"), ctypes.byref(ls), _stream(stream))
        _check(st, self._h)
        return out, lists

    # ---- training
    def saved_bytes(self, B: int) -> int:
        """Bytes of the activations rmx_block_forward_train keeps for B samples."""
        return int(self._lib.rmx_saved_bytes(self._h, B))

    def forward_train(self, X, weights: dict, out=None, saved=None, stream=None):
        """The forward pass that also keeps what the backward needs: returns (out, saved),
        saved a device byte tensor to hand to backward() unchanged."""
        import torch
        c = self.cfg
        B = X.shape[0]
        _ptr(X, "X", self.dtype, (B, c.T, c.D))
        if out is None:
            out = torch.empty((B, c.D), dtype=torch.float32, device=X.device)
        _ptr(out, "out", torch.float32, (B, c.D))
        nbytes = self.saved_bytes(B)
        if saved is None:
            saved = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=X.device)
        _ptr(saved, "saved", torch.uint8)
        ws = self._weights(weights)
        _check(self._lib.rmx_block_forward_train(self._h, _ptr(X, "X"), B, ctypes.byref(ws), c.L, c.k,
                                                 _ptr(out, "out"), _ptr(saved, "saved"), saved.numel(),
                                                 _stream(stream)), self._h)
        return out, saved

    def backward(self, X, weights: dict, saved, g_out, dX=None, grads: dict | None = None, stream=None):
        """Gradients of a loss whose gradient with respect to out is g_out [B, D] (fp32):
        returns (dX [B, T, D] fp32, {"W1": dW1, ..., "ln2_b": dln2_b} fp32, summed over the
        batch).  X, weights and saved are those of the forward_train call."""
        import torch
        c = self.cfg
        B = X.shape[0]
        kD = c.k * c.D
        _ptr(X, "X", self.dtype, (B, c.T, c.D))
        _ptr(g_out, "g_out", torch.float32, (B, c.D))
        _ptr(saved, "saved", torch.uint8)
        shapes = {"W1": (c.L, c.T, c.D, kD), "b1": (c.L, c.T, kD), "W2": (c.L, c.T, kD, c.D),
                  "b2": (c.L, c.T, c.D), "ln1_g": (c.L, c.D), "ln1_b": (c.L, c.D), "ln2_g": (c.L, c.D),
                  "ln2_b": (c.L, c.D)}
        if dX is None:
            dX = torch.empty((B, c.T, c.D), dtype=torch.float32, device=X.device)
        _ptr(dX, "dX", torch.float32, (B, c.T, c.D))
        if grads is None:
            grads = {n: torch.empty(shp, dtype=torch.float32, device=X.device) for n, shp in shapes.items()}
        g = rmx_grads()
        for n in GRAD_NAMES:
            setattr(g, "d" + n, _ptr(grads[n], "d" + n, torch.float32, shapes[n]))
        ws = self._weights(weights)
        _check(self._lib.rmx_block_backward(self._h, _ptr(X, "X"), B, ctypes.byref(ws), c.L, c.k,
                                            _ptr(saved, "saved"), saved.numel(), _ptr(g_out, "g_out"),
                                            _ptr(dX, "dX"), ctypes.byref(g), _stream(stream)), self._h)
        return dX, grads

    # ---- kernel timing
    def profile_enable(self, on: bool = True):
        _check(self._lib.rmx_profile_enable(self._h, int(on)), self._h)

    def profile_reset(self):
        _check(self._lib.rmx_profile_reset(self._h), self._h)

    def profile_read(self) -> dict:
        ms = (ctypes.c_double * KERNEL_COUNT)()
        n = (ctypes.c_int64 * KERNEL_COUNT)()
        dropped = ctypes.c_int64()
        _check(self._lib.rmx_profile_read(self._h, ms, n, ctypes.byref(dropped)), self._h)
        out = {}
        for i in range(KERNEL_COUNT):
            if n[i]:
                out[self._lib.rmx_kernel_name(i).decode()] = {"total_ms": ms[i], "launches": n[i],
                                                              "avg_ms": ms[i] / n[i]}
        out["_dropped"] = dropped.value
        return out


def token_mix(X, Y=None, stream=None):
    """Y[b, h, t*q + r] = X[b, t, h*q + r] on the GPU (the library's mixing kernel)."""
    import torch
    lib = load_library()
    B, T, D = X.shape
    code = _dtype_code(X.dtype)
    _ptr(X, "X")
    if Y is None:
        Y = torch.empty_like(X)
    _ptr(Y, "Y", X.dtype, X.shape)
    _check(lib.rmx_token_mix(_ptr(X, "X"), _ptr(Y, "Y"), B, T, D, code, _stream(stream)))
    return Y


def tokenize(E, Wp, bp=None, X=None, stream=None):
    """X[b, t] = E[b, t*d:(t+1)*d] @ Wp[t] + bp[t] on the GPU (the library's tokenisation
    projection); E [B, T*d], Wp [T, d, D], bp [T, D] or None; returns X [B, T, D]."""
    import torch
    lib = load_library()
    T, d, D = Wp.shape
    B = E.shape[0]
    code = _dtype_code(E.dtype)
    _ptr(E, "E", E.dtype, (B, T * d))
    _ptr(Wp, "Wp", E.dtype)
    if bp is not None:
        _ptr(bp, "bp", E.dtype, (T, D))
    if X is None:
        X = torch.empty((B, T, D), dtype=E.dtype, device=E.device)
    _ptr(X, "X", E.dtype, (B, T, D))
    _check(lib.rmx_tokenize(_ptr(E, "E"), _ptr(Wp, "Wp"), _ptr(bp, "bp"), _ptr(X, "X"), B, T, d, D, code,
                            _stream(stream)))
    return X


def upload(inputs, device="cuda"):
    """Device copies of a synth.Inputs: (X, weights dict), in the workload's dtype."""
    import torch
    dt = _torch_dtype(_dtype_code(inputs.cfg.dtype))

    def dev(a):
        return torch.from_numpy(a).to(device=device).to(dt).contiguous()

    w = {n: dev(getattr(inputs, n)) for n in ("W1", "b1", "W2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")}
    for n, a in inputs.moe.items():
        w[n] = dev(a)
    for n, a in inputs.attn.items():
        w[n] = dev(a)
    return dev(inputs.X), w
