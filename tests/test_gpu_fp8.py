"""GPU parity of the fp8 (e4m3 + fp32 block scales) path against the oracle.

The gathered codes and their scales are bit-exact; the kernel's e4m3
quantisation of the SwiGLU output is checked bit-exactly against the oracle's
codec applied to the kernel's own fp32 values, with the quantisation decision
(value / scale, then round to nearest even) taken in fp32 on both sides; Y
within 3e-2 relative Frobenius of the oracle that quantises H the same way.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_cases import check_y, fill_x_perm, problem_of, run_layer, to_gpu

pytestmark = pytest.mark.gpu

FP8 = {
    "fp8_small_segments": moe_synth.make_config("tiny", T=1024, d=256, f=256, E_global=16, k=4, e_begin=0, e_end=8,
                                                dtype="fp8_e4m3", num_segments=8, seed=21),
    "fp8_multi_band": moe_synth.make_config("tiny", T=1024, d=384, f=256, E_global=4, k=2, dtype="fp8_e4m3",
                                            seed=22),
}


def _run(cfg, sched="interleaved", **kw):
    import expert_grouped_gemm_amd as moe
    inp = moe_synth.generate(cfg)
    g = to_gpu(inp)
    p = problem_of(cfg, sched=sched, **kw)
    Y, Y32, ws = run_layer(p, g)
    moe.check_workspace(p, ws)
    return inp, g, p, Y, Y32, ws


@pytest.mark.parametrize("name", list(FP8))
def test_fp8_dispatch_codes_and_scales_exact(name):
    import expert_grouped_gemm_amd as moe
    cfg = FP8[name]
    inp, g, p, Y, Y32, ws = _run(cfg)
    ref = oracle.moe_layer(inp, cfg)
    v = {k: t.cpu() for k, t in moe.workspace_views(p, ws).items()}
    fused_scale = v["x_perm_scale"].clone()       # written by the fused call's scatter
    v["x_perm"] = fill_x_perm(p, g, ws)["x_perm"].cpu()
    A = ref["A"]
    np.testing.assert_array_equal(v["topk_idx"].numpy(), ref["topk_idx"])
    np.testing.assert_array_equal(v["row_src"].numpy()[:A], ref["row_src"])
    np.testing.assert_array_equal(v["row_dst"].numpy()[:A], ref["row_dst"])
    np.testing.assert_array_equal(v["tok_off"].numpy(), ref["tok_off"])
    tok = ref["row_src"] // cfg.k
    np.testing.assert_array_equal(v["x_perm"].numpy()[:A], inp["X"].numpy()[tok])
    xs = inp["X_scale"].numpy()
    np.testing.assert_array_equal(v["x_perm_scale"].numpy()[:, :A], xs[tok // 128].T)
    np.testing.assert_array_equal(fused_scale.numpy()[:, :A], xs[tok // 128].T)


@pytest.mark.parametrize("tiles", ["narrow", "wide"])
@pytest.mark.parametrize("name", list(FP8))
def test_fp8_h_quantiser_bit_exact(name, tiles):
    """Narrow Linear-1 tiles cover half a 128-column block each (the second one
    quantises it), wide tiles a whole block."""
    import expert_grouped_gemm_amd as moe
    cfg = FP8[name]
    inp, g, p, Y, Y32, ws = _run(cfg, tiles=tiles, keep_h_f32=True)
    v = {k: t.cpu() for k, t in moe.workspace_views(p, ws).items()}
    A = int(v["meta"][0])
    hf = v["h_f32"].numpy()[:A].astype(np.float32)
    blocks = hf.reshape(A, cfg.f // 128, 128)
    amax = np.abs(blocks).max(axis=2).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q32 = (blocks / scale[:, :, None]).astype(np.float32)          # fp32 quotient, as the kernel
    codes = oracle.f64_to_e4m3_bits(q32.astype(np.float64)).reshape(A, cfg.f)
    np.testing.assert_array_equal(v["h_scale"].numpy()[:, :A].T, scale)
    np.testing.assert_array_equal(v["h"].numpy()[:A], codes)


@pytest.mark.parametrize("tiles", ["narrow", "wide"])
@pytest.mark.parametrize("sched", ["separate", "expert_wave", "interleaved"])
@pytest.mark.parametrize("name", list(FP8))
def test_fp8_layer_y_parity(name, sched, tiles):
    cfg = FP8[name]
    inp, g, p, Y, Y32, ws = _run(cfg, sched=sched, tiles=tiles)
    ref = oracle.moe_layer(inp, cfg)
    stats = check_y(Y.float().cpu().numpy(), ref["Y"], fp8=True, label=f"{name}/{sched}")
    # the same quantisation on both sides: far inside the 3e-2 budget
    assert stats["rel_fro"] < 5e-3, stats


def test_fp8_schedule_invariance_bitwise():
    cfg = FP8["fp8_multi_band"]
    g = to_gpu(moe_synth.generate(cfg))
    base, _, _ = run_layer(problem_of(cfg, sched="separate"), g, want_fp32=False)
    for kw in (dict(sched="expert_wave"), dict(sched="interleaved"), dict(sched="interleaved", lead_D=1, grid=8),
               dict(sched="separate", keep_h_f32=True), dict(sched="separate", tiles="narrow"),
               dict(sched="separate", tiles="wide"), dict(sched="interleaved", tiles="wide"),
               dict(sched="separate", tiles="narrow", band_major=True)):
        Y, _, _ = run_layer(problem_of(cfg, **kw), g, want_fp32=False)
        assert torch.equal(Y.view(torch.int16), base.view(torch.int16)), kw


def test_fp8_fused_schedules_never_read_stale_h():
    """As for bf16: poisoned workspace (0xFF: e4m3 NaN codes, NaN fp32 staging)
    before every fused call; Y must equal the separate-launch Y bit for bit."""
    import expert_grouped_gemm_amd as moe
    cfg = FP8["fp8_small_segments"]
    g = to_gpu(moe_synth.generate(cfg))
    base, _, _ = run_layer(problem_of(cfg, sched="separate"), g, want_fp32=False)
    for kw in (dict(sched="interleaved"), dict(sched="interleaved", lead_D=1), dict(sched="expert_wave"),
               dict(sched="interleaved", tiles="wide"), dict(sched="expert_wave", tiles="wide")):
        p = problem_of(cfg, **kw)
        ws = moe.alloc_workspace(p)
        for _ in range(3):
            ws.fill_(0xFF)
            Y, _, _ = run_layer(p, g, ws=ws, want_fp32=False)
            moe.check_workspace(p, ws)
            assert torch.equal(Y.view(torch.int16), base.view(torch.int16)), kw
