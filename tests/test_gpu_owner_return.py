"""GPU parity of the owner-aligned return path (Cui et al., Sections 3.2-3.3)
through the C ABI: the host plan, the padded gather, the grouped expert GEMM
run on the padded layout (offsets = expert_off, row_dst = identity) and the
segment copy into the receive buffer.

Checks: the padded rows bit-exact against the gathered X rows and zeros; the
receive buffer bit-exact against the fused path's expert outputs (the same
kernels compute each output row with the same K order wherever the row sits
in a band) and, on the small workloads, within tolerance of the fp64 oracle;
padding rows never reach the receive buffer.
"""
import numpy as np
import pytest
import torch

import expert_grouped_gemm_amd as moe
import moe_synth
import oracle
from moe_cases import fill_x_perm, problem_of, run_layer, to_gpu
from oracle import owner_layout as ol

pytestmark = pytest.mark.gpu


def padded_problem(p, R):
    """p with a workspace row capacity that holds the R padded rows."""
    q = moe.Problem.from_buffer_copy(p)
    q.row_capacity = max(R, moe.row_capacity(p))
    return q


def _owner_return(p, g, idx, local, tb, x):
    plan = moe.owner_plan(p, idx, local, tb, x)
    R = plan["R"]
    p = padded_problem(p, R)
    cap = moe.row_capacity(p)
    row_src = torch.from_numpy(plan["row_src"]).cuda()
    fp8 = p.dtype == moe.DTYPE["fp8_e4m3"]
    X_pad = torch.empty((R, p.d), dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
    X_pad_scale = torch.empty((p.d // 128, cap), dtype=torch.float32, device="cuda") if fp8 else None
    moe.owner_gather(p, g["X"], g.get("X_scale"), row_src, X_pad, X_pad_scale)
    O_pad = torch.empty((R, p.d), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(p)
    moe.expert_forward(p, X_pad, X_pad_scale, torch.from_numpy(plan["expert_off"]).cuda(),
                       torch.arange(R, dtype=torch.int32, device="cuda"), g["W1"], g.get("W1_scale"), g["W2"],
                       g.get("W2_scale"), O_pad, ws)
    recv = torch.full((plan["recv_rows"], p.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.segment_copy(p, O_pad, torch.from_numpy(plan["segments"]).cuda().contiguous(), recv)
    torch.cuda.synchronize()
    return plan, X_pad, recv


def _fused_outputs_by_assignment(p, ws):
    """Expert output row of every local assignment id, from the fused path's
    workspace (combine_buf slot row_dst[r] holds assignment row_src[r])."""
    v = moe.workspace_views(p, ws)
    A = int(v["meta"][0].item())
    rs = v["row_src"][:A].cpu().numpy()
    rd = v["row_dst"][:A].cpu().numpy()
    buf = v["combine_buf"][:A].cpu().numpy()
    out = {int(a): buf[int(s)] for a, s in zip(rs, rd)}
    return out, v["topk_idx"].cpu().numpy()


SMALL = {
    "share_s4": (moe_synth.make_config("tiny", T=512, d=256, f=256, E_global=8, k=4, e_begin=0, e_end=4,
                                       num_segments=4, seed=21), 1, 32, 2),
    "ragged_s8": (moe_synth.make_config("tiny", T=1024, d=384, f=128, E_global=16, k=4, e_begin=5, e_end=11,
                                        num_segments=8, seed=22), 0, 16, 3),
    "zipf_s2": (moe_synth.make_config("tiny", T=2048, d=256, f=256, E_global=16, k=4, e_begin=0, e_end=8,
                                      zipf_s=1.2, num_segments=2, seed=23), 1, 64, 2),
    # every expert local: any padding takes the layout past T * min(k, E_l),
    # so the workspace is sized by row_capacity
    "all_local_s4": (moe_synth.make_config("tiny", T=512, d=256, f=256, E_global=8, k=2, e_begin=0, e_end=8,
                                           num_segments=4, seed=26), 1, 32, 2),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_owner_return_small(name):
    cfg, local, tb, x = SMALL[name]
    print(f"owner return {name} local={local} tb={tb} x={x}", flush=True)
    inp = moe_synth.generate(cfg)
    ref = oracle.moe_layer(inp, cfg)
    g = to_gpu(inp)
    p = problem_of(cfg, sched="separate")
    _, _, ws = run_layer(p, g)
    fused, idx = _fused_outputs_by_assignment(p, ws)
    np.testing.assert_array_equal(idx, ref["topk_idx"])
    plan, X_pad, recv = _owner_return(p, g, idx, local, tb, x)
    if name == "all_local_s4":
        assert plan["R"] > cfg.cap
    # padded gather: X rows bit-exact, zero rows where row_src = -1
    rs = plan["row_src"]
    xs = inp["X"].view(torch.int16).numpy()
    xp = X_pad.view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(xp[rs >= 0], xs[rs[rs >= 0] // cfg.k])
    assert not np.any(xp[rs < 0])
    # receive buffer: bit-exact against the fused path, by the layout-free definition
    got = recv.cpu().numpy()
    want = ol.segment_return(idx, cfg.e_begin, cfg.e_end, cfg.num_segments, lambda a: fused[a])
    np.testing.assert_array_equal(got, want)
    # and within tolerance of the oracle's fp64 expert outputs
    slot = np.empty(cfg.T * cfg.k, dtype=np.int64)
    slot[ref["tok_list"]] = np.arange(ref["A"])
    o_ref = ol.segment_return(idx, cfg.e_begin, cfg.e_end, cfg.num_segments,
                              lambda a: ref["combine_buf"][slot[a]])
    err = np.linalg.norm(got - o_ref) / np.linalg.norm(o_ref)
    assert err <= 5e-3, err


def test_owner_return_deepseek_share_full_size():
    # The DeepSeek-style share at full size with eight owner ranks (token t on
    # rank t mod 8), this GPU rank 0, tb_M = 32, middle segments of 2 bands.
    cfg = moe_synth.make_config("deepseek_share_bf16", num_segments=8)
    print("owner return deepseek_share_bf16 S=8 local=0 tb=32 x=2", flush=True)
    g = moe_synth.generate(cfg, device="cuda")
    p = problem_of(cfg, sched="separate")
    _, _, ws = run_layer(p, g)
    fused, idx = _fused_outputs_by_assignment(p, ws)
    plan, X_pad, recv = _owner_return(p, g, idx, 0, 32, 2)
    A = len(fused)
    assert plan["recv_rows"] == A
    assert plan["R"] - A <= cfg.E_local * 7 * 31
    got = recv.cpu().numpy()
    # layout-free expected order, vectorised: region s, then expert, then assignment id
    flat = idx.reshape(-1)
    a_all = np.arange(flat.size)
    local = (flat >= cfg.e_begin) & (flat < cfg.e_end)
    a_loc = a_all[local]
    key = np.lexsort((a_loc, flat[a_loc], (a_loc // cfg.k) % 8))
    order = a_loc[key]
    want = np.stack([fused[int(a)] for a in order])
    np.testing.assert_array_equal(got, want)


def _overlapped(p, X, g, plan, ws, grid=0):
    """Gather, then the signalling GEMM on the launch stream and the waiting
    segment copier on a second stream (default priority). The GEMM is
    enqueued first: where the runtime maps both streams onto one hardware
    queue, the copier then runs after the GEMM instead of holding it back."""
    R = plan["R"]
    p = padded_problem(p, R)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    row_src = torch.from_numpy(plan["row_src"]).cuda()
    X_pad = torch.empty((R, p.d), dtype=torch.bfloat16, device="cuda")
    O_pad = torch.full((R, p.d), float("nan"), dtype=torch.float32, device="cuda")
    recv = torch.full((plan["recv_rows"], p.d), float("nan"), dtype=torch.float32, device="cuda")
    row_done = torch.zeros((R + 31) // 32, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    segs = torch.from_numpy(plan["segments"]).cuda().contiguous()
    eo = torch.from_numpy(plan["expert_off"]).cuda()
    iota = torch.arange(R, dtype=torch.int32, device="cuda")
    moe.owner_gather(p, X, None, row_src, X_pad, None, main)
    ev = torch.cuda.Event()
    ev.record(main)
    side.wait_event(ev)
    moe.expert_forward_signal(p, X_pad, None, eo, iota, g["W1"], None, g["W2"], None, O_pad, row_done, ws,
                              stream=main)
    moe.segment_copy_wait(p, O_pad, R, segs, recv, row_done, err, grid, stream=side)
    main.wait_stream(side)
    torch.cuda.synchronize()
    return recv, int(err.item()), row_done


@pytest.mark.parametrize("name", ["share_s4", "ragged_s8", "all_local_s4"])
def test_overlapped_copy_matches_stream_ordered(name):
    cfg, local, tb, x = SMALL[name]
    print(f"overlapped owner return {name}", flush=True)
    inp = moe_synth.generate(cfg)
    g = to_gpu(inp)
    p = problem_of(cfg, sched="separate")
    _, _, ws = run_layer(p, g)
    idx = moe.workspace_views(p, ws)["topk_idx"].cpu().numpy()
    plan = moe.owner_plan(p, idx, local, tb, x)
    ws2 = moe.alloc_workspace(padded_problem(p, plan["R"]))
    # two calls in a row, the second on other token values (no stale rows may be copied)
    X2 = moe_synth.generate(cfg, seed=cfg.seed + 100)["X"].cuda()
    for X in (g["X"], X2):
        g2 = dict(g, X=X)
        want = _owner_return(p, g2, idx, local, tb, x)[2].cpu().numpy()
        recv, err, row_done = _overlapped(p, X, g, plan, ws2, grid=8)
        assert err == 0
        R = plan["R"]
        full = np.minimum(32, R - 32 * np.arange(len(row_done))) * p.d
        np.testing.assert_array_equal(row_done.cpu().numpy(), full)
        np.testing.assert_array_equal(recv.cpu().numpy(), want)


def test_overlapped_copy_deepseek_share_full_size():
    cfg = moe_synth.make_config("deepseek_share_bf16", num_segments=8)
    print("overlapped owner return deepseek_share_bf16 S=8 local=0 tb=32 x=2", flush=True)
    g = moe_synth.generate(cfg, device="cuda")
    p = problem_of(cfg, sched="separate")
    _, _, ws = run_layer(p, g)
    idx = moe.workspace_views(p, ws)["topk_idx"].cpu().numpy()
    plan, _, want = _owner_return(p, g, idx, 0, 32, 2)
    recv, err, _ = _overlapped(p, g["X"], g, plan, moe.alloc_workspace(padded_problem(p, plan["R"])))
    assert err == 0
    torch.testing.assert_close(recv, want, rtol=0, atol=0)


def test_copier_wait_timeout_is_reported():
    # No GEMM runs, so no block is ever complete: the first segment's bounded
    # wait gives up, sets the error word, and every segment is skipped.
    cfg, local, tb, x = SMALL["share_s4"]
    print("copier timeout path", flush=True)
    p = problem_of(cfg, sched="separate")
    rng = np.random.default_rng(0)
    idx = rng.integers(0, cfg.E_global, size=(cfg.T, cfg.k)).astype(np.int32)
    plan = moe.owner_plan(p, idx, local, tb, x)
    R = plan["R"]
    O_pad = torch.zeros((R, p.d), dtype=torch.float32, device="cuda")
    recv = torch.full((plan["recv_rows"], p.d), float("nan"), dtype=torch.float32, device="cuda")
    row_done = torch.zeros((R + 31) // 32, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    segs = torch.from_numpy(plan["segments"]).cuda().contiguous()
    moe.segment_copy_wait(p, O_pad, R, segs, recv, row_done, err, grid=4)
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    assert torch.isnan(recv).all()


def test_owner_return_fp8():
    # e4m3 codes with 128x128 block scales: padded codes and row scales
    # bit-exact, receive buffer bit-exact against the fused fp8 path.
    cfg = moe_synth.make_config("tiny", T=512, d=256, f=256, E_global=8, k=4, e_begin=0, e_end=4,
                                dtype="fp8_e4m3", num_segments=4, seed=24)
    print("owner return fp8 small S=4 local=2 tb=32 x=2", flush=True)
    inp = moe_synth.generate(cfg)
    g = to_gpu(inp)
    p = problem_of(cfg, sched="separate")
    _, _, ws = run_layer(p, g)
    fused, idx = _fused_outputs_by_assignment(p, ws)
    plan = moe.owner_plan(p, idx, 2, 32, 2)
    R, cap = plan["R"], cfg.cap
    assert R <= cap  # the gather's scale rows are laid out with the problem's row capacity
    row_src = torch.from_numpy(plan["row_src"]).cuda()
    X_pad = torch.empty((R, p.d), dtype=torch.uint8, device="cuda")
    X_pad_scale = torch.full((p.d // 128, cap), -7.0, dtype=torch.float32, device="cuda")
    moe.owner_gather(p, g["X"], g["X_scale"], row_src, X_pad, X_pad_scale)
    torch.cuda.synchronize()
    rs = plan["row_src"]
    xs = inp["X"].numpy()
    sc = inp["X_scale"].numpy()
    got_x = X_pad.cpu().numpy()
    np.testing.assert_array_equal(got_x[rs >= 0], xs[rs[rs >= 0] // cfg.k])
    assert not np.any(got_x[rs < 0])
    got_s = X_pad_scale.cpu().numpy()
    tok = np.maximum(rs, 0) // cfg.k
    want_s = np.where(rs[None, :] >= 0, sc[tok // 128].T, 1.0)
    np.testing.assert_array_equal(got_s[:, :R], want_s)
    assert np.all(got_s[:, R:] == -7.0)
    plan2, _, recv = _owner_return(p, g, idx, 2, 32, 2)
    want = ol.segment_return(idx, cfg.e_begin, cfg.e_end, cfg.num_segments, lambda a: fused[a])
    np.testing.assert_array_equal(recv.cpu().numpy(), want)


def test_owner_return_fp8_deepseek_share_full_size():
    cfg = moe_synth.CONFIGS["deepseek_share_fp8"]
    print("owner return deepseek_share_fp8 S=8 local=0 tb=32 x=2", flush=True)
    g = moe_synth.generate(cfg, device="cuda")
    p = problem_of(cfg, sched="separate")
    _, _, ws = run_layer(p, g)
    fused, idx = _fused_outputs_by_assignment(p, ws)
    plan, _, recv = _owner_return(p, g, idx, 0, 32, 2)
    flat = idx.reshape(-1)
    a_loc = np.nonzero((flat >= cfg.e_begin) & (flat < cfg.e_end))[0]
    order = a_loc[np.lexsort((a_loc, flat[a_loc], (a_loc // cfg.k) % 8))]
    want = np.stack([fused[int(a)] for a in order])
    np.testing.assert_array_equal(recv.cpu().numpy(), want)


@pytest.mark.parametrize("sched", ["separate", "expert_wave", "interleaved"])
def test_signal_counts_every_output_element(sched):
    # In every schedule (including the interleaved tail of narrow Linear-2
    # tiles), the signalling GEMM counts each stored output element once per
    # 32-row block, and writes the same rows as the plain GEMM.
    cfg = moe_synth.make_config("tiny", T=1000, d=384, f=384, E_global=16, k=4, e_begin=3, e_end=11,
                                num_segments=4, seed=25)
    print(f"signal counts {sched}", flush=True)
    g = to_gpu(moe_synth.generate(cfg))
    p = problem_of(cfg, sched=sched)
    _, _, ws = run_layer(p, g)
    v = fill_x_perm(p, g, ws)
    A = int(v["meta"][0].item())
    R = A
    iota = torch.arange(max(R, 1), dtype=torch.int32, device="cuda")
    O_plain = torch.full((R, p.d), float("nan"), dtype=torch.float32, device="cuda")
    O_sig = torch.full((R, p.d), float("nan"), dtype=torch.float32, device="cuda")
    row_done = torch.zeros((R + 31) // 32, dtype=torch.int32, device="cuda")
    ws2 = moe.alloc_workspace(p)
    moe.expert_forward(p, v["x_perm"], None, v["offsets"], iota, g["W1"], None, g["W2"], None, O_plain, ws2)
    moe.expert_forward_signal(p, v["x_perm"], None, v["offsets"], iota, g["W1"], None, g["W2"], None, O_sig,
                              row_done, ws2)
    torch.cuda.synchronize()
    moe.check_workspace(p, ws2)
    full = np.minimum(32, R - 32 * np.arange(len(row_done))) * p.d
    np.testing.assert_array_equal(row_done.cpu().numpy(), full)
    torch.testing.assert_close(O_sig, O_plain, rtol=0, atol=0)
