"""The boundary's optional parts on the GPU: moe_layer_forward's routing and
dispatch outputs, MOE_FLAG_FP32_Y_DEBUG, and the bf16 combine buffer
(MOE_FLAG_BF16_COMBINE_BUF), a measured variant whose distance to the oracle
is reported here."""
import numpy as np
import pytest
import torch

import expert_grouped_gemm_amd as moe
import moe_synth
import oracle
from moe_cases import bf16_ulp, check_y, problem_of, run_layer, to_gpu

pytestmark = pytest.mark.gpu

CFG = moe_synth.make_config("tiny", T=1000, d=384, f=384, E_global=16, k=4, e_begin=3, e_end=11, num_segments=4,
                            seed=11)


def test_layer_forward_optional_outputs():
    print("[boundary] optional outputs", flush=True)
    inp = moe_synth.generate(CFG)
    g = to_gpu(inp)
    p = problem_of(CFG, sched="separate")
    Y0, _, ws0 = run_layer(p, g, want_fp32=False)
    v0 = moe.workspace_views(p, ws0)
    cap, El = moe.row_capacity(p), CFG.E_local
    outs = dict(topk_idx=torch.full((CFG.T, CFG.k), -3, dtype=torch.int32, device="cuda"),
                topk_w=torch.full((CFG.T, CFG.k), -3.0, dtype=torch.float32, device="cuda"),
                counts=torch.full((El,), -3, dtype=torch.int32, device="cuda"),
                offsets=torch.full((El + 1,), -3, dtype=torch.int32, device="cuda"),
                row_src=torch.full((cap,), -3, dtype=torch.int32, device="cuda"))
    ws = moe.alloc_workspace(p)
    ws.fill_(0xA5)
    Y = torch.empty_like(Y0)
    moe.layer_forward(p, g["X"], None, g["logits"], g["W1"], None, g["W2"], None, Y, None, ws, **outs)
    torch.cuda.synchronize()
    moe.check_workspace(p, ws)
    assert torch.equal(Y, Y0)
    A = int(v0["meta"][0])
    for key, t in outs.items():
        want = v0[key]
        if key == "row_src":
            assert torch.equal(t[:A], want[:A]) and torch.all(t[A:] == -3)
        else:
            assert torch.equal(t, want), key
    # the regions the outputs replace were not written
    v = moe.workspace_views(p, ws)
    for key in outs:
        assert torch.all(v[key].view(torch.uint8) == 0xA5), key


def test_fp32_y_debug_flag():
    print("[boundary] fp32 Y flag", flush=True)
    g = to_gpu(moe_synth.generate(CFG))
    p = problem_of(CFG, sched="separate")
    Y0, Y32_0, _ = run_layer(p, g)
    pf = problem_of(CFG, sched="separate", fp32_y=True)
    Y, Y32, _ = run_layer(pf, g)
    assert torch.equal(Y, Y0) and torch.equal(Y32, Y32_0)
    with pytest.raises(moe.MoEError):
        run_layer(pf, g, want_fp32=False)


@pytest.mark.parametrize("sched", ["separate", "interleaved"])
def test_bf16_combine_buffer(sched):
    """The combine buffer in bf16: each expert output is rounded once more
    before the weighted sum. Relative Frobenius error stays within 5e-3; the
    max-abs criterion is reported (the extra rounding costs about a bf16 ulp
    of each output, which the 1e-2 rms bound need not absorb)."""
    print(f"[boundary] bf16 combine buffer, {sched}", flush=True)
    inp = moe_synth.generate(CFG)
    ref = oracle.moe_layer(inp, CFG)
    g = to_gpu(inp)
    p = problem_of(CFG, sched=sched, bf16_combine_buf=True)
    Y, Y32, ws = run_layer(p, g)
    moe.check_workspace(p, ws)
    y, r = Y.float().cpu().numpy().astype(np.float64), ref["Y"]
    rel = np.linalg.norm(y - r) / np.linalg.norm(r)
    rms = np.sqrt(np.mean(r ** 2))
    allow = np.maximum(np.abs(y - r) - bf16_ulp(r), 0.0).max() / rms
    strict32 = np.abs(Y32.cpu().numpy().astype(np.float64) - r).max() / rms
    print(f"[boundary] bf16 combine buffer {sched}: rel_fro={rel:.3e} maxabs_ulp_allow/rms={allow:.3e} "
          f"maxabs_fp32/rms={strict32:.3e}", flush=True)
    assert rel <= 5e-3
    # the buffer holds exactly the bf16 rounding of the fp32 path's expert outputs
    p32 = problem_of(CFG, sched=sched)
    _, _, ws32 = run_layer(p32, g)
    A = int(moe.workspace_views(p32, ws32)["meta"][0])
    b16 = moe.workspace_views(p, ws)["combine_buf"][:A]
    b32 = moe.workspace_views(p32, ws32)["combine_buf"][:A]
    assert torch.equal(b16, b32.to(torch.bfloat16))
