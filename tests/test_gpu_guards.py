"""Device-side argument checks (arguments that live in device memory, where
the host cannot validate them before the launch). Each case feeds a bad
argument that the kernels themselves must catch: nothing outside the
buffers is written, the outputs the check protects are left untouched, and
moe_check_workspace reports MOE_ERR_INVALID_ARGUMENT. A good call on the same
workspace afterwards is clean and correct.

Every bad value here is one the kernels bound-check before any access (the
planning kernel rejects the offsets before a tile exists, the epilogue
tests each row_dst before its store, the combine each slot range before its
loads, the scatter each position before its store), so no case can reach
memory outside its buffers."""
import numpy as np
import pytest
import torch

import expert_grouped_gemm_amd as moe
import moe_synth
import oracle
from moe_cases import check_y, fill_x_perm, problem_of, run_layer, to_gpu

pytestmark = pytest.mark.gpu

CFG = moe_synth.make_config("tiny", T=256, d=256, f=256, E_global=8, k=2, e_begin=0, e_end=4, seed=31)


def _expect_invalid(p, ws):
    with pytest.raises(moe.MoEError) as ei:
        moe.check_workspace(p, ws)
    assert ei.value.status == 1
    moe.check_workspace(p, ws)  # the report clears the words


@pytest.mark.parametrize("sched", ["separate", "interleaved"])
def test_offsets_past_capacity_store_nothing(sched):
    print(f"[guards] offsets past capacity, {sched}", flush=True)
    inp = moe_synth.generate(CFG)
    g = to_gpu(inp)
    p = problem_of(CFG, sched=sched)
    cap = moe.row_capacity(p)
    _, _, ws = run_layer(p, g)                      # a good call first: the workspace holds real values
    v = fill_x_perm(p, g, ws)
    x_perm = v["x_perm"].clone()
    row_dst = v["row_dst"].clone()
    h_before = v["h"].clone()
    C = torch.full((cap, CFG.d), 7.0, dtype=torch.float32, device="cuda")
    El = CFG.E_local
    for bad in ([0, 10, 20, 30, cap + 1], [0, 50, 40, 60, 70], [-1, 10, 20, 30, 40]):
        offsets = torch.tensor(bad, dtype=torch.int32, device="cuda")
        assert offsets.numel() == El + 1
        moe.expert_forward(p, x_perm, None, offsets, row_dst, g["W1"], None, g["W2"], None, C, ws)
        torch.cuda.synchronize()
        _expect_invalid(p, ws)
        assert torch.all(C == 7.0), bad
        # bit patterns: the rows past A hold whatever the workspace held, NaNs included
        assert torch.equal(v["h"].view(torch.int16), h_before.view(torch.int16)), bad
    # the same workspace, good offsets again
    moe.expert_forward(p, x_perm, None, v["offsets"], row_dst, g["W1"], None, g["W2"], None, C, ws)
    torch.cuda.synchronize()
    moe.check_workspace(p, ws)
    A = int(v["meta"][0])
    torch.testing.assert_close(C[:A], v["combine_buf"][:A], rtol=0, atol=0)


def test_row_dst_outside_capacity_is_not_stored():
    print("[guards] row_dst outside capacity", flush=True)
    g = to_gpu(moe_synth.generate(CFG))
    p = problem_of(CFG, sched="separate")
    cap = moe.row_capacity(p)
    _, _, ws = run_layer(p, g)
    v = fill_x_perm(p, g, ws)
    A = int(v["meta"][0])
    row_dst = v["row_dst"].clone()
    bad_rows = [0, A // 2, A - 1]
    row_dst[bad_rows] = torch.tensor([cap, -5, 1 << 30], dtype=torch.int32, device="cuda")
    C = torch.full((cap, CFG.d), 7.0, dtype=torch.float32, device="cuda")
    moe.expert_forward(p, v["x_perm"], None, v["offsets"], row_dst, g["W1"], None, g["W2"], None, C, ws)
    torch.cuda.synchronize()
    _expect_invalid(p, ws)
    good = v["row_dst"][[r for r in range(A) if r not in bad_rows]].long()
    torch.testing.assert_close(C[good], v["combine_buf"][good], rtol=0, atol=0)
    skipped = v["row_dst"][bad_rows].long()
    assert torch.all(C[skipped] == 7.0)


def test_combine_slot_range_outside_capacity_gives_nan_rows():
    print("[guards] combine slot range", flush=True)
    g = to_gpu(moe_synth.generate(CFG))
    p = problem_of(CFG, sched="separate")
    cap = moe.row_capacity(p)
    Y0, _, ws = run_layer(p, g, want_fp32=False)
    v = moe.workspace_views(p, ws)
    tok_off = v["tok_off"].clone()
    tok_off[5] = cap + 3          # rows 4 and 5 get ranges past the buffer / reversed
    Y = torch.empty_like(Y0)
    moe.combine(p, v["combine_buf"], tok_off, v["comb_w"], Y)
    torch.cuda.synchronize()
    assert torch.isnan(Y[4].float()).all() and torch.isnan(Y[5].float()).all()
    keep = [q for q in range(CFG.T) if q not in (4, 5)]
    assert torch.equal(Y[keep], Y0[keep])


def test_dispatch_past_capacity_is_reported():
    """A caller's topk_idx that lists local expert 0 twice for every token:
    2 T local assignments against a row capacity of T (E_l = 1). The
    scatter stores only rows that fit, the gather nothing, the expert GEMM
    refuses the offsets, and the combine's ranges give NaN rows."""
    print("[guards] dispatch past capacity", flush=True)
    cfg = CFG.replace(e_begin=0, e_end=1)
    g = to_gpu(moe_synth.generate(cfg))
    p = problem_of(cfg, sched="separate")
    cap = moe.row_capacity(p)
    assert cap == cfg.T
    ws = moe.alloc_workspace(p)
    v = moe.workspace_views(p, ws)
    idx = torch.zeros((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.full((cfg.T, cfg.k), 0.5, dtype=torch.float32, device="cuda")
    X_perm = torch.full((cap, cfg.d), 3.0, dtype=torch.bfloat16, device="cuda")
    row_src = torch.full((cap,), -9, dtype=torch.int32, device="cuda")
    moe.dispatch(p, g["X"], None, idx, w, v["counts"], v["offsets"], row_src, v["row_dst"], v["tok_off"],
                 v["comb_w"], X_perm, None, ws)
    torch.cuda.synchronize()
    assert int(v["offsets"][-1]) == 2 * cfg.T
    _expect_invalid(p, ws)
    assert torch.all(X_perm.float() == 3.0)            # the gather copied nothing
    rs = row_src.cpu().numpy()
    assert np.all((rs >= 0) & (rs < cfg.T * cfg.k))    # every row that fits is a valid assignment
    C = torch.full((cap, cfg.d), 7.0, dtype=torch.float32, device="cuda")
    moe.expert_forward(p, X_perm, None, v["offsets"], v["row_dst"], g["W1"], None, g["W2"], None, C, ws)
    torch.cuda.synchronize()
    _expect_invalid(p, ws)
    assert torch.all(C == 7.0)
    Y = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    moe.combine(p, C, v["tok_off"], v["comb_w"], Y)
    torch.cuda.synchronize()
    tok_off = v["tok_off"].cpu().numpy()
    bad = tok_off[1:] > cap
    assert bad.any()
    assert torch.isnan(Y[torch.as_tensor(np.flatnonzero(bad), device="cuda")].float()).all()
    # the same workspace with a valid routing: clean and correct
    inp = moe_synth.generate(cfg)
    ref = oracle.moe_layer(inp, cfg)
    Yg, Y32, _ = run_layer(p, g, ws=ws)
    moe.check_workspace(p, ws)
    check_y(Yg.float().cpu().numpy(), ref["Y"], Y32.cpu().numpy(), label="after guard")
