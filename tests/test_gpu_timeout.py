"""The readiness-wait timeout path, forced from the host (a flag that makes
the fused schedules' readiness target unreachable): the bounded wait gives
up, the kernels exit normally, moe_check_workspace reports MOE_ERR_DEADLOCK,
and the next ordinary call on the same workspace reports nothing and is
correct again."""
import pytest
import torch

import moe_synth
import oracle
from moe_cases import check_y, problem_of, run_layer, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sched", ["interleaved", "expert_wave"])
def test_forced_wait_timeout_is_reported_and_cleared(sched):
    import expert_grouped_gemm_amd as moe
    cfg = moe_synth.make_config("tiny", T=512, d=128, f=256, E_global=4, k=2, seed=51)
    inp = moe_synth.generate(cfg)
    g = to_gpu(inp)
    bad = problem_of(cfg, sched=sched)
    bad.flags |= moe.FLAG_TEST_WAIT_TIMEOUT
    ws = moe.alloc_workspace(bad)
    run_layer(bad, g, ws=ws, want_fp32=False)
    with pytest.raises(moe.MoEError) as err:
        moe.check_workspace(bad, ws)
    assert err.value.status == 5  # MOE_ERR_DEADLOCK
    good = problem_of(cfg, sched=sched)
    Y, Y32, _ = run_layer(good, g, ws=ws)
    moe.check_workspace(good, ws)
    check_y(Y.float().cpu().numpy(), oracle.moe_layer(inp, cfg)["Y"], Y32.cpu().numpy(), label=sched)
