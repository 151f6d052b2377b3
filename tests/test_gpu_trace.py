"""Per-tile timing records of the expert GEMM (trace=True).

What the records must satisfy whatever the timing: tracing changes no output
bit; every row band's Linear-1 tiles cover its f SwiGLU columns, and its
Linear-2 tiles its d output columns, exactly once (the widths may differ from
tile to tile where the separate schedule splits its last round); each record's
clock readings are ordered; a workgroup runs its tiles one after another; and
no Linear-2 tile of a row band passes its readiness wait before every Linear-1
tile of that band has finished its K loop (the separate schedule: before every
Linear-1 tile has ended, since the second launch starts after the first).
"""
import numpy as np
import pytest
import torch

import moe_synth
from moe_cases import problem_of, run_layer, to_gpu

pytestmark = pytest.mark.gpu

CFGS = {
    "bf16_multi_band": moe_synth.make_config("tiny", T=2048, d=512, f=512, E_global=8, k=2, seed=41),
    "fp8_multi_band": moe_synth.make_config("tiny", T=1024, d=384, f=256, E_global=4, k=2, dtype="fp8_e4m3",
                                            seed=42),
}


def _covered(spans, total):
    spans = sorted(spans)
    pos = 0
    for a, b in spans:
        if a != pos:
            return False
        pos = b
    return pos == total


@pytest.mark.parametrize("kw", [dict(sched="separate"), dict(sched="separate", grid=6),
                                dict(sched="expert_wave"), dict(sched="interleaved"),
                                dict(sched="interleaved", tiles="narrow"), dict(sched="auto")], ids=str)
@pytest.mark.parametrize("name", list(CFGS))
def test_tile_trace(name, kw):
    import expert_grouped_gemm_amd as moe
    cfg = CFGS[name]
    g = to_gpu(moe_synth.generate(cfg))
    base, _, _ = run_layer(problem_of(cfg, **kw), g, want_fp32=False)
    p = problem_of(cfg, trace=True, **kw)
    ws = moe.alloc_workspace(p)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    Y, _, ws = run_layer(p, g, ws=ws, want_fp32=False)
    e1.record()
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), base.view(torch.int16))
    assert 1e6 <= moe.lib().moe_tile_clock_hz() <= 1e10
    moe.check_workspace(p, ws)
    tr = moe.tile_trace(p, ws)
    nb = int(moe.workspace_views(p, ws)["meta"][1])
    assert nb > 1
    kind, band, n, nnb = tr["kind"], tr["band"], tr["n"], tr["nnb"]
    assert set(np.unique(kind)) == {1, 2}
    assert np.all((nnb == 2) | (nnb == 4))
    assert np.all((band >= 0) & (band < nb))
    for b in range(nb):
        l1, l2 = (kind == 1) & (band == b), (kind == 2) & (band == b)
        assert _covered([(int(x) * w * 32, (int(x) + 1) * w * 32) for x, w in zip(n[l1], nnb[l1])], cfg.f), b
        assert _covered([(int(x) * w * 64, (int(x) + 1) * w * 64) for x, w in zip(n[l2], nnb[l2])], cfg.d), b
    ts, tr_, tm, te = tr["t_start"], tr["t_ready"], tr["t_main_end"], tr["t_end"]
    assert np.all(ts <= tr_) and np.all(tr_ <= tm) and np.all(tm <= te)
    # the tiles ran inside the call's event-timed interval
    assert te.max() - ts.min() <= e0.elapsed_time(e1) * 1e3 * 1.01
    for w in np.unique(tr["wg"]):
        sel = np.flatnonzero(tr["wg"] == w)
        order = sel[np.argsort(ts[sel], kind="stable")]
        assert np.all(ts[order[1:]] >= te[order[:-1]]), w
    if moe.schedule_of(p) == "separate":  # two launches (auto resolves to them)
        assert ts[kind == 2].min() >= te[kind == 1].max()
    else:
        for b in range(nb):
            assert tr_[(kind == 2) & (band == b)].min() >= tm[(kind == 1) & (band == b)].max(), b
