"""Degenerate shares against the oracle, in every schedule and both tile
widths:

* no local assignment at all (the local experts are never in any token's
  top-k), bf16 and fp8: A = 0, no row band reaches the expert GEMMs, and Y
  is exactly zero;
* a single token routed to a single expert (T = 1, k = 1, E = 1);
* one token per destination segment with a local share that gets only some
  of them.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_cases import check_y, problem_of, run_layer, to_gpu

pytestmark = pytest.mark.gpu

SCHEDS = ["separate", "expert_wave", "interleaved", "auto"]


def _cases():
    # local experts 6 and 7 are pushed out of every top-2
    no_local = moe_synth.make_config("tiny", T=300, d=128, f=256, E_global=8, k=2, e_begin=6, e_end=8, seed=31)
    inp = moe_synth.generate(no_local)
    inp["logits"][:, 6:8] = -1.0e4
    yield "no_local", no_local, inp
    no_local_fp8 = moe_synth.make_config("tiny", T=256, d=256, f=256, E_global=8, k=2, e_begin=6, e_end=8,
                                         dtype="fp8_e4m3", seed=34)
    inp = moe_synth.generate(no_local_fp8)
    inp["logits"][:, 6:8] = -1.0e4
    yield "no_local_fp8", no_local_fp8, inp
    single = moe_synth.make_config("tiny", T=1, d=128, f=128, E_global=1, k=1, e_begin=0, e_end=1, seed=32)
    yield "single_token", single, moe_synth.generate(single)
    seg = moe_synth.make_config("tiny", T=8, d=256, f=128, E_global=4, k=2, e_begin=1, e_end=3, num_segments=8,
                                seed=33)
    yield "token_per_segment", seg, moe_synth.generate(seg)


CASES = {name: (cfg, inp) for name, cfg, inp in _cases()}


@pytest.mark.parametrize("tiles", ["narrow", "wide"])
@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_share(name, sched, tiles):
    import expert_grouped_gemm_amd as moe
    cfg, inp = CASES[name]
    ref = oracle.moe_layer(inp, cfg)
    p = problem_of(cfg, sched=sched, tiles=tiles)
    Y, Y32, ws = run_layer(p, to_gpu(inp))
    moe.check_workspace(p, ws)
    v = {k: t.cpu() for k, t in moe.workspace_views(p, ws).items()}
    A = ref["A"]
    assert int(v["meta"][0]) == A
    np.testing.assert_array_equal(v["topk_idx"].numpy(), ref["topk_idx"])
    np.testing.assert_array_equal(v["tok_off"].numpy(), ref["tok_off"])
    np.testing.assert_array_equal(v["row_src"].numpy()[:A], ref["row_src"])
    if name.startswith("no_local"):
        assert A == 0 and int(v["meta"][1]) == 0
        assert torch.count_nonzero(Y.float()).item() == 0 and torch.count_nonzero(Y32).item() == 0
    else:
        assert A > 0
        check_y(Y.float().cpu().numpy(), ref["Y"], Y32.cpu().numpy(), label=f"{name}/{sched}/{tiles}")


# Router widths: ceil(E / 64) logits per lane = 2, 8 and 16 (E = 1024 and
# k = 16 are the largest the library accepts); the whole layer on a local
# share, with routing and dispatch compared bit for bit.
WIDE_E = {
    "E100_k8": moe_synth.make_config("tiny", T=256, d=128, f=128, E_global=100, k=8, e_begin=10, e_end=60, seed=41),
    "E300_k16": moe_synth.make_config("tiny", T=192, d=128, f=128, E_global=300, k=16, e_begin=0, e_end=300,
                                      seed=42),
    "E1024_k16": moe_synth.make_config("tiny", T=128, d=128, f=128, E_global=1024, k=16, e_begin=512, e_end=1024,
                                       num_segments=2, seed=43),
}


@pytest.mark.parametrize("name", list(WIDE_E))
def test_router_widths_and_large_expert_counts(name):
    import expert_grouped_gemm_amd as moe
    cfg = WIDE_E[name]
    inp = moe_synth.generate(cfg)
    ref = oracle.moe_layer(inp, cfg)
    p = problem_of(cfg, sched="auto")
    Y, Y32, ws = run_layer(p, to_gpu(inp))
    moe.check_workspace(p, ws)
    v = {k: t.cpu() for k, t in moe.workspace_views(p, ws).items()}
    A = ref["A"]
    np.testing.assert_array_equal(v["topk_idx"].numpy(), ref["topk_idx"])
    np.testing.assert_allclose(v["topk_w"].numpy(), ref["topk_w"], rtol=2e-6, atol=1e-7)
    for key in ("counts", "offsets", "tok_off"):
        np.testing.assert_array_equal(v[key].numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(v["row_src"].numpy()[:A], ref["row_src"])
    np.testing.assert_array_equal(v["row_dst"].numpy()[:A], ref["row_dst"])
    check_y(Y.float().cpu().numpy(), ref["Y"], Y32.cpu().numpy(), label=name)


def test_dispatch_scan_of_a_long_token_batch():
    """T = 100000: each of the scan's 16 wavefronts owns 6272 output rows,
    far more than its registers hold, so the scan walks its segment in
    passes, and the last segment is ragged. Routing and the whole dispatch,
    from the fused call and from the component calls, bit for bit against
    the oracle."""
    import expert_grouped_gemm_amd as moe
    cfg = moe_synth.make_config("tiny", T=100000, d=128, f=128, E_global=64, k=4, e_begin=8, e_end=40,
                                num_segments=4, seed=61)
    print("[degenerate] T=100000 dispatch", flush=True)
    inp = moe_synth.generate(cfg)
    idx, w, _ = oracle.route_topk(inp["logits"].numpy(), cfg.k)
    ref = oracle.dispatch(idx, w, cfg.e_begin, cfg.e_end, cfg.num_segments)
    A = ref["A"]
    g = to_gpu(inp)
    p = problem_of(cfg, sched="auto")
    _, _, ws = run_layer(p, g, want_fp32=False)
    moe.check_workspace(p, ws)
    v = {k: t.cpu() for k, t in moe.workspace_views(p, ws).items() if k not in ("x_perm", "h", "combine_buf")}
    np.testing.assert_array_equal(v["topk_idx"].numpy(), idx)
    for key in ("counts", "offsets", "tok_off"):
        np.testing.assert_array_equal(v[key].numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(v["row_src"].numpy()[:A], ref["row_src"])
    np.testing.assert_array_equal(v["row_dst"].numpy()[:A], ref["row_dst"])
    # the component dispatch's scan kernel on the same routing
    ws2 = moe.alloc_workspace(p)
    v2 = moe.workspace_views(p, ws2)
    moe.dispatch(p, g["X"], None, v["topk_idx"].cuda(), v["topk_w"].cuda(), v2["counts"], v2["offsets"],
                 v2["row_src"], v2["row_dst"], v2["tok_off"], v2["comb_w"], v2["x_perm"], None, ws2)
    torch.cuda.synchronize()
    moe.check_workspace(p, ws2)
    for key in ("counts", "offsets", "tok_off"):
        np.testing.assert_array_equal(v2[key].cpu().numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(v2["row_src"].cpu().numpy()[:A], ref["row_src"])
