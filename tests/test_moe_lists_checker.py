"""CPU check of the routing-list checker the GPU tests use (tests/parity.py
check_moe_lists): lists built from the definition pass, and each plausible mistake of a
routing kernel (a wrong order, a missing or extra row, a shifted offset, a wrong tile count,
a stale inverse map, a wrong gate value) is caught."""
import numpy as np
import pytest

from tests.parity import check_moe_lists


def _lists_from_gates(g, tile=256):
    """Routing lists written out from their definition (group gi = t*E + e lists the b
    with g[b, t, e] > 0 in ascending order, as token rows t*B + b)."""
    L, B, T, E = g.shape
    G = T * E
    out = {k: [] for k in ("group_start", "rows", "row_gate", "pos", "tile_start")}
    for n in range(L):
        gs, rows, rg, tiles = [0], [], [], [0]
        pos = np.full((G, B), -1, dtype=np.int32)
        for t in range(T):
            for e in range(E):
                for b in range(B):
                    if g[n, b, t, e] > 0:
                        pos[t * E + e, b] = len(rows)
                        rows.append(t * B + b)
                        rg.append(g[n, b, t, e])
                gs.append(len(rows))
                tiles.append(tiles[-1] + (gs[-1] - gs[-2] + tile - 1) // tile)
        pad = G * B - len(rows)
        out["group_start"].append(np.array(gs, dtype=np.int32))
        out["rows"].append(np.array(rows + [-7] * pad, dtype=np.int32))
        out["row_gate"].append(np.array(rg + [np.nan] * pad, dtype=np.float32))
        out["pos"].append(pos.reshape(-1))
        out["tile_start"].append(np.array(tiles, dtype=np.int32))
    return {k: np.stack(v) for k, v in out.items()}


def _gates(L=2, B=300, T=3, E=4, seed=0):
    g = np.random.default_rng(seed).standard_normal((L, B, T, E)).astype(np.float32)
    return np.maximum(g, 0.0)


def test_definition_passes():
    g = _gates()
    frac = check_moe_lists(_lists_from_gates(g), g)
    assert all(0.4 < f < 0.6 for f in frac)


def _plant(kind, lists, g):
    n, gi = 1, 5
    gs = lists["group_start"][n]
    lo, hi = gs[gi], gs[gi + 1]
    if kind == "order":
        lists["rows"][n, lo], lists["rows"][n, lo + 1] = lists["rows"][n, lo + 1], lists["rows"][n, lo]
    elif kind == "row":
        lists["rows"][n, hi - 1] += 1
    elif kind == "offset":
        lists["group_start"][n, gi + 1] += 1
    elif kind == "tiles":
        lists["tile_start"][n, -1] += 1
    elif kind == "pos":
        b = lists["rows"][n, lo] % g.shape[1]
        lists["pos"][n].reshape(-1, g.shape[1])[gi, b] = -1
    elif kind == "gate":
        lists["row_gate"][n, lo] = np.nextafter(lists["row_gate"][n, lo], np.float32(2))
    elif kind == "dropped":
        b = lists["rows"][n, lo] % g.shape[1]
        g[n, b, gi // g.shape[3], gi % g.shape[3]] = 0.0   # the list keeps a row whose gate is 0


@pytest.mark.parametrize("kind", ["order", "row", "offset", "tiles", "pos", "gate", "dropped"])
def test_planted_mistakes_are_caught(kind):
    g = _gates()
    lists = _lists_from_gates(g)
    _plant(kind, lists, g)
    with pytest.raises(AssertionError):
        check_moe_lists(lists, g)
