"""GPU parity of the W4A8 path (e4m3 activations with fp32 block scales,
MXFP4 weights: E2M1 codes and E8M0 block scales) against the oracle, which
decodes the same bits from the MX definition.

Routing and dispatch are bit-exact as for fp8; the e4m3 quantisation of the
SwiGLU output is bit-exact against the oracle's codec applied to the kernel's
own fp32 values; Y within 3e-2 relative Frobenius of the oracle that
quantises H the same way (and, as the two sides apply identical roundings,
far inside it). At full size, the DeepSeek-style share with MXFP4 weights is
compared on one sampled row in every 256-row band of every expert.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_cases import check_y, problem_of, run_layer, to_gpu

pytestmark = pytest.mark.gpu

W4 = {
    "w4_small_segments": moe_synth.make_config("tiny", T=1024, d=256, f=256, E_global=16, k=4, e_begin=0, e_end=8,
                                               dtype="w4a8_mxfp4", num_segments=8, seed=51),
    "w4_multi_band": moe_synth.make_config("tiny", T=1024, d=384, f=256, E_global=4, k=2, dtype="w4a8_mxfp4",
                                           seed=52),
    "w4_share": moe_synth.make_config("tiny", T=512, d=512, f=384, E_global=32, k=8, e_begin=4, e_end=12,
                                      dtype="w4a8_mxfp4", num_segments=4, seed=53),
}


def _run(cfg, sched="separate", **kw):
    import expert_grouped_gemm_amd as moe
    inp = moe_synth.generate(cfg)
    g = to_gpu(inp)
    p = problem_of(cfg, sched=sched, **kw)
    Y, Y32, ws = run_layer(p, g)
    moe.check_workspace(p, ws)
    return inp, g, p, Y, Y32, ws


@pytest.mark.parametrize("tiles", ["narrow", "wide"])
@pytest.mark.parametrize("sched", ["separate", "expert_wave", "interleaved"])
@pytest.mark.parametrize("name", list(W4))
def test_w4a8_layer_y_parity(name, sched, tiles):
    print(f"[w4a8] {name} {sched} {tiles}", flush=True)
    cfg = W4[name]
    inp, g, p, Y, Y32, ws = _run(cfg, sched=sched, tiles=tiles)
    ref = oracle.moe_layer(inp, cfg)
    stats = check_y(Y.float().cpu().numpy(), ref["Y"], fp8=True, label=f"{name}/{sched}/{tiles}")
    assert stats["rel_fro"] < 5e-3, stats


@pytest.mark.parametrize("tiles", ["narrow", "wide"])
def test_w4a8_h_quantiser_bit_exact(tiles):
    import expert_grouped_gemm_amd as moe
    cfg = W4["w4_multi_band"]
    print(f"[w4a8] H quantiser {tiles}", flush=True)
    inp, g, p, Y, Y32, ws = _run(cfg, tiles=tiles, keep_h_f32=True)
    v = {k: t.cpu() for k, t in moe.workspace_views(p, ws).items()}
    A = int(v["meta"][0])
    hf = v["h_f32"].numpy()[:A].astype(np.float32)
    blocks = hf.reshape(A, cfg.f // 128, 128)
    amax = np.abs(blocks).max(axis=2).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q32 = (blocks / scale[:, :, None]).astype(np.float32)
    codes = oracle.f64_to_e4m3_bits(q32.astype(np.float64)).reshape(A, cfg.f)
    np.testing.assert_array_equal(v["h_scale"].numpy()[:, :A].T, scale)
    np.testing.assert_array_equal(v["h"].numpy()[:A], codes)
    # and the fp32 SwiGLU values themselves against the oracle's, per row
    ref = oracle.moe_layer(inp, cfg, h_mode=None)
    X = oracle.decode_x(inp, cfg)
    offs, rs = ref["offsets"], ref["row_src"]
    for e in range(cfg.E_local):
        rows = np.arange(offs[e], offs[e + 1])
        if rows.size == 0:
            continue
        W1e, _ = oracle.decode_expert_weights(inp, cfg, e)
        h = X[rs[rows] // cfg.k] @ W1e.T
        act = h[:, :cfg.f] / (1 + np.exp(-h[:, :cfg.f])) * h[:, cfg.f:]
        err = np.linalg.norm(hf[rows] - act) / np.linalg.norm(act)
        assert err < 1e-5, (e, err)


def test_w4a8_schedule_invariance_bitwise():
    cfg = W4["w4_share"]
    print("[w4a8] schedule invariance", flush=True)
    g = to_gpu(moe_synth.generate(cfg))
    base, _, _ = run_layer(problem_of(cfg, sched="separate"), g, want_fp32=False)
    for kw in (dict(sched="expert_wave"), dict(sched="interleaved"), dict(sched="interleaved", lead_D=1, grid=8),
               dict(sched="separate", tiles="narrow"), dict(sched="separate", tiles="wide", band_major=True)):
        Y, _, _ = run_layer(problem_of(cfg, **kw), g, want_fp32=False)
        assert torch.equal(Y.view(torch.int16), base.view(torch.int16)), kw


@pytest.mark.parametrize("sched", ["auto", "interleaved"])
def test_w4a8_deepseek_share_full_size(sched):
    """The DeepSeek-style share with MXFP4 weights at full size, in the
    benchmark's launch configuration and the interleaved schedule: routing and
    dispatch bit-exact, Y on one sampled row per 256-row band of every expert."""
    import expert_grouped_gemm_amd as moe
    from test_gpu_fullsize import BAND, band_sample, bands_of_rows
    cfg = moe_synth.CONFIGS["deepseek_share_w4a8"]
    print(f"[w4a8] full size {sched}", flush=True)
    g = moe_synth.generate(cfg, device="cuda")
    p = problem_of(cfg, sched=sched)
    Y, _, ws = run_layer(p, g, want_fp32=False)
    moe.check_workspace(p, ws)
    host = {k: t.cpu() for k, t in g.items()}
    idx, w, _ = oracle.route_topk(host["logits"].numpy(), cfg.k)
    disp = oracle.dispatch(idx, w, cfg.e_begin, cfg.e_end, cfg.num_segments)
    v = moe.workspace_views(p, ws)
    A = disp["A"]
    np.testing.assert_array_equal(v["topk_idx"].cpu().numpy(), idx)
    np.testing.assert_array_equal(v["offsets"].cpu().numpy(), disp["offsets"])
    np.testing.assert_array_equal(v["row_src"].cpu().numpy()[:A], disp["row_src"])
    tokens, rows = band_sample(disp["offsets"], disp["row_src"], cfg.k, np.random.default_rng(13))
    sampled = np.flatnonzero(np.isin(disp["row_src"] // cfg.k, tokens))
    offs = disp["offsets"]
    assert bands_of_rows(offs, sampled) == {(e, b) for e in range(offs.size - 1)
                                           for b in range(-(-int(offs[e + 1] - offs[e]) // BAND))}
    ref = oracle.moe_layer(host, cfg, tokens=tokens)
    q = oracle.y_row_of_token(tokens, cfg.T, cfg.num_segments)
    stats = check_y(Y.float().cpu().numpy()[q], ref["Y"][q], fp8=True, label=f"w4a8 full/{sched}")
    print(f"[w4a8] full size {sched}: {stats}", flush=True)
    assert stats["rel_fro"] < 5e-3, stats
