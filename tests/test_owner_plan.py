"""The library's owner-aligned plan (moe_owner_plan, host code in the C ABI)
against the oracle (Cui et al., Sections 3.2-3.3), bit-exact: small random
routings and the routings of the four large workload shapes, several tile
heights, segment widths and local ranks. No GPU is needed."""
import numpy as np
import pytest

import expert_grouped_gemm_amd as moe
import oracle
from oracle import owner_layout as ol


def _routing(T, E, k, seed, zipf_s=0.0):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    if zipf_s:
        L += (-zipf_s * np.log(np.arange(1, E + 1))).astype(np.float32)[None, :]
    idx, _, _ = oracle.route_topk(L, k)
    return idx.astype(np.int32)


def _compare(idx, T, E, k, eb, ee, S, local, tb, x):
    p = moe.make_problem(T, 128, 128, E, k, eb, ee, num_segments=S)
    got = moe.owner_plan(p, idx, local, tb, x)
    lay = ol.owner_aligned_layout(idx, eb, ee, S, local, tb)
    assert got["row_src"].tolist() == lay["row_src"].tolist()
    assert got["expert_off"].tolist() == lay["expert_off"].tolist()
    b = got["bands"]
    for col, key in enumerate(("band_expert", "band_dest", "band_row", "band_valid", "band_recv_off")):
        assert b[:, col].tolist() == lay[key].tolist(), key
    assert got["schedule"].tolist() == ol.remote_first_schedule(lay).tolist()
    seg = ol.transfer_segments(lay, x)
    s = got["segments"]
    for col, key in enumerate(("src_row", "rows", "dst_row", "dest")):
        assert s[:, col].tolist() == seg[key].tolist(), key
    assert got["recv_start"].tolist() == [0] + np.cumsum(lay["recv_rows"]).tolist()
    assert got["remote_bands"] == int(np.sum(lay["band_dest"] != local))
    return got, lay


@pytest.mark.parametrize("T,E,k,eb,ee,S,local,tb,x", [
    (40, 8, 2, 0, 4, 4, 0, 4, 2), (64, 16, 4, 4, 10, 8, 3, 8, 3), (96, 6, 3, 1, 6, 3, 2, 5, 1),
    (33, 4, 4, 0, 4, 1, 0, 1, 2), (128, 32, 8, 0, 8, 8, 7, 32, 2), (256, 8, 2, 0, 8, 2, 1, 16, 4)])
def test_plan_matches_oracle_small(T, E, k, eb, ee, S, local, tb, x):
    if T % S:
        pytest.skip("T must be a multiple of S")
    _compare(_routing(T, E, k, T * 7 + E), T, E, k, eb, ee, S, local, tb, x)


@pytest.mark.parametrize("name,T,E,k,eb,ee,zipf", [
    ("deepseek_share", 4096, 256, 8, 0, 32, 0.0), ("dit_skewed", 32768, 64, 4, 0, 64, 1.2),
    ("mixtral", 16384, 8, 2, 0, 8, 0.0)])
@pytest.mark.parametrize("tb", [32, 256])
def test_plan_matches_oracle_workload_shapes(name, T, E, k, eb, ee, zipf, tb):
    idx = _routing(T, E, k, 11, zipf)
    got, lay = _compare(idx, T, E, k, eb, ee, 8, 0, tb, 2)
    A = int(np.sum((idx >= eb) & (idx < ee)))
    assert got["recv_rows"] == A
    assert got["R"] - A <= (ee - eb) * 7 * (tb - 1)            # Section 4.5 bound per expert, summed


def test_plan_sizes_only_and_errors():
    T, E, k = 64, 8, 2
    idx = _routing(T, E, k, 3)
    p = moe.make_problem(T, 128, 128, E, k, 0, 8, num_segments=4)
    L = moe.lib()
    import ctypes
    z = moe.OwnerPlanSizes()
    a = np.ascontiguousarray(idx)
    assert L.moe_owner_plan(ctypes.byref(p), a.ctypes.data, 0, 16, 2, None, 0, None, None, None, None, 0, None,
                            ctypes.byref(z)) == 0
    assert z.recv_rows == T * k and z.R >= T * k
    buf = np.zeros(1, np.int32)
    st = L.moe_owner_plan(ctypes.byref(p), a.ctypes.data, 0, 16, 2, buf.ctypes.data, 1, buf.ctypes.data,
                          buf.ctypes.data, buf.ctypes.data, buf.ctypes.data, 1, buf.ctypes.data, ctypes.byref(z))
    assert st == 3                                                   # MOE_ERR_WORKSPACE_TOO_SMALL
    for local, tb, x in ((4, 16, 2), (-1, 16, 2), (0, 0, 2), (0, 16, 0), (0, 5000, 1)):
        assert L.moe_owner_plan(ctypes.byref(p), a.ctypes.data, local, tb, x, None, 0, None, None, None, None, 0,
                                None, ctypes.byref(z)) == 1
    pf = moe.make_problem(128, 128, 128, E, k, 0, 8, num_segments=4, dtype="fp8_e4m3")
    assert L.moe_owner_gather(ctypes.byref(pf), 16, None, 16, 1, 16, None, None) == 1   # fp8 needs scales
    assert L.moe_owner_gather(ctypes.byref(p), 16, 16, 16, 1, 16, None, None) == 1      # bf16 takes none
    cap = 128 * 2
    assert L.moe_owner_gather(ctypes.byref(pf), 16, 16, 16, cap + 1, 16, 16, None) == 2  # fp8 rows beyond cap
    assert L.moe_segment_copy(ctypes.byref(p), None, 4, None, 1, None, 4, None) == 1
    rd = np.zeros(4, np.int32)
    assert L.moe_segment_copy_wait(ctypes.byref(pf), 16, 64, 16, 1, 16, 64, rd.ctypes.data, 4, 16, 0, None) == 2
