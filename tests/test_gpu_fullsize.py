"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (the run-time schedule choice, default tiles and grid) and in
the interleaved schedule.

Routing, counts, offsets and the whole dispatch permutation are compared
bit-exactly with the oracle. Y is compared on sampled output rows that the
oracle computes token by token. The sample holds, for every local expert,
one row at a random position inside each of its 256-row bands (the GEMM's
row bands, so every tile of both grouped launches produces at least one
compared element: a row's Y element n comes from the Linear-2 tile holding
column n, and its H from every Linear-1 tile of the band) plus the expert's
last row (the ragged tail), and tokens without a local expert, whose rows
must be exactly zero. The test asserts that every band was sampled.
fp8 also reports (and bounds by the same 3e-2) the distance to the oracle
that keeps H in fp32, i.e. without the e4m3 quantisation of the intermediate.
"""
import functools

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_cases import check_y, fill_x_perm, problem_of, run_layer

pytestmark = pytest.mark.gpu

FULL = ["deepseek_share_bf16", "dit_skewed", "mixtral", "deepseek_share_fp8"]
BAND = 256  # rows per GEMM row band


def band_sample(offsets, row_src, k, rng):
    """Rows: one random row per 256-row band of each expert plus the expert's
    last row. Returns (tokens, band ids (expert, band) covered)."""
    rows = []
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for b0 in range(lo, hi, BAND):
            rows.append(int(rng.integers(b0, min(b0 + BAND, hi))))
        if hi > lo:
            rows.append(hi - 1)
    rows = np.asarray(sorted(set(rows)), dtype=np.int64)
    return np.unique(row_src[rows] // k), rows


def bands_of_rows(offsets, rows):
    e = np.searchsorted(offsets, rows, side="right") - 1
    return set(zip(e.tolist(), ((rows - offsets[e]) // BAND).tolist()))


@functools.lru_cache(maxsize=1)
def reference(name):
    """Inputs (generated on the GPU, seeded), the oracle's routing/dispatch and
    its Y on the band sample: computed once per workload for both schedules."""
    cfg = moe_synth.CONFIGS[name]
    g = moe_synth.generate(cfg, device="cuda")
    host = {k: t.cpu() for k, t in g.items()}
    idx, w, _ = oracle.route_topk(host["logits"].numpy(), cfg.k)
    disp = oracle.dispatch(idx, w, cfg.e_begin, cfg.e_end, cfg.num_segments)
    rng = np.random.default_rng(11)
    tokens, rows = band_sample(disp["offsets"], disp["row_src"], cfg.k, rng)
    has = np.zeros(cfg.T, bool)
    has[disp["row_src"] // cfg.k] = True
    without = np.flatnonzero(~has)[:4]
    ref = oracle.moe_layer(host, cfg, tokens=np.concatenate([tokens, without]))
    pure = oracle.moe_layer(host, cfg, h_mode=None, tokens=tokens) if cfg.dtype == "fp8_e4m3" else None
    return cfg, g, idx, w, disp, tokens, without, ref, pure


@pytest.mark.parametrize("sched", ["auto", "interleaved"])
@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name, sched):
    import expert_grouped_gemm_amd as moe
    cfg, g, idx, w, disp, tokens, without, ref, pure = reference(name)
    print(f"[fullsize] {name}/{sched}: {tokens.size} sampled tokens", flush=True)
    p = problem_of(cfg, sched=sched)
    Y, Y32, ws = run_layer(p, g)
    moe.check_workspace(p, ws)
    v = {k: t.cpu() for k, t in moe.workspace_views(p, ws).items() if k not in ("x_perm", "h", "h_f32", "combine_buf")}
    np.testing.assert_array_equal(v["topk_idx"].numpy(), idx)
    np.testing.assert_allclose(v["topk_w"].numpy(), w, rtol=2e-6, atol=1e-7)
    A = disp["A"]
    assert int(v["meta"][0]) == A
    for key in ("counts", "offsets", "tok_off"):
        np.testing.assert_array_equal(v[key].numpy(), disp[key], err_msg=key)
    np.testing.assert_array_equal(v["row_src"].numpy()[:A], disp["row_src"])
    np.testing.assert_array_equal(v["row_dst"].numpy()[:A], disp["row_dst"])

    # every row band of every expert has a sampled row
    sampled_rows = np.flatnonzero(np.isin(disp["row_src"] // cfg.k, tokens))
    offs = disp["offsets"]
    all_bands = {(e, b) for e in range(offs.size - 1) for b in range(-(-int(offs[e + 1] - offs[e]) // BAND))}
    assert bands_of_rows(offs, sampled_rows) == all_bands

    q = oracle.y_row_of_token(tokens, cfg.T, cfg.num_segments)
    Yall = Y.float().cpu().numpy()
    if without.size:
        qz = oracle.y_row_of_token(without, cfg.T, cfg.num_segments)
        assert np.all(Yall[qz] == 0.0)
    fp8 = cfg.dtype == "fp8_e4m3"
    stats = check_y(Yall[q], ref["Y"][q], None if fp8 else Y32.cpu().numpy()[q], fp8=fp8, label=f"{name}/{sched}")
    if fp8:
        pq = pure["Y"][q]
        stats["rel_fro_vs_fp32_h"] = float(np.linalg.norm(Yall[q] - pq) / np.linalg.norm(pq))
        assert stats["rel_fro_vs_fp32_h"] <= 3e-2, stats
    print(f"[fullsize] {name}/{sched}: {stats}", flush=True)

    # the component dispatch's gathered X rows of the sampled bands are exact copies
    xp = fill_x_perm(p, g, ws)["x_perm"]
    got = xp[torch.as_tensor(sampled_rows, device="cuda")].cpu()
    want = g["X"][torch.as_tensor(disp["row_src"][sampled_rows] // cfg.k, device="cuda")].cpu()
    assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))
