"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (the run-time schedule choice, default tiles and grid) and in
the interleaved schedule.

Routing, counts, offsets and the whole dispatch permutation are compared
bit-exactly with the oracle; Y is compared on sampled output rows the oracle
computes one token at a time (tokens with local experts, plus tokens without,
whose rows must be exactly zero).
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_cases import check_y, problem_of, run_layer

pytestmark = pytest.mark.gpu

FULL = ["deepseek_share_bf16", "dit_skewed", "mixtral", "deepseek_share_fp8"]


@pytest.mark.parametrize("sched", ["auto", "interleaved"])
@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name, sched):
    import expert_grouped_gemm_amd as moe
    cfg = moe_synth.CONFIGS[name]
    g = moe_synth.generate(cfg, device="cuda")
    p = problem_of(cfg, sched=sched)
    Y, Y32, ws = run_layer(p, g)
    moe.check_workspace(p, ws)
    v = {k: t.cpu() for k, t in moe.workspace_views(p, ws).items() if k not in ("x_perm", "h", "h_f32", "combine_buf")}
    host = {k: t.cpu() for k, t in g.items() if k in ("logits",)}
    idx, w, cg = oracle.route_topk(host["logits"].numpy(), cfg.k)
    np.testing.assert_array_equal(v["topk_idx"].numpy(), idx)
    np.testing.assert_allclose(v["topk_w"].numpy(), w, rtol=2e-6, atol=1e-7)
    disp = oracle.dispatch(idx, w, cfg.e_begin, cfg.e_end, cfg.num_segments)
    A = disp["A"]
    assert int(v["meta"][0]) == A
    for key in ("counts", "offsets", "tok_off"):
        np.testing.assert_array_equal(v[key].numpy(), disp[key], err_msg=key)
    np.testing.assert_array_equal(v["row_src"].numpy()[:A], disp["row_src"])
    np.testing.assert_array_equal(v["row_dst"].numpy()[:A], disp["row_dst"])

    # sampled Y rows
    rng = np.random.default_rng(0)
    has = np.zeros(cfg.T, bool)
    has[disp["row_src"] // cfg.k] = True
    with_local = rng.choice(np.flatnonzero(has), size=min(12, int(has.sum())), replace=False)
    without = np.flatnonzero(~has)[:4]
    tokens = np.concatenate([with_local, without]).astype(np.int64)
    inp_host = {k: t.cpu() for k, t in g.items()}
    ref = oracle.moe_layer(inp_host, cfg, tokens=tokens)
    q = oracle.y_row_of_token(tokens, cfg.T, cfg.num_segments)
    Yh = Y.float().cpu().numpy()[q]
    if without.size:
        qz = oracle.y_row_of_token(without, cfg.T, cfg.num_segments)
        assert np.all(Y.float().cpu().numpy()[qz] == 0.0)
    check_y(Yh, ref["Y"][q], None if cfg.dtype == "fp8_e4m3" else Y32.cpu().numpy()[q],
            fp8=cfg.dtype == "fp8_e4m3", label=f"{name}/{sched}")
    # x_perm rows of the sampled tokens were gathered exactly
    xp = moe.workspace_views(p, ws)["x_perm"]
    rows = np.flatnonzero(np.isin(disp["row_src"] // cfg.k, with_local))[:32]
    got = xp[torch.as_tensor(rows, device="cuda")].cpu()
    want = g["X"][torch.as_tensor(disp["row_src"][rows] // cfg.k, device="cuda")].cpu()
    assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))
