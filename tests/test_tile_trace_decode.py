"""tile_trace() decodes moe_tile_record_t as moe_mi355x.h documents it (no
GPU: records are written into a host workspace by hand, and the clock rate
the library would report is replaced by a fixed 100 MHz)."""
import numpy as np
import torch

import expert_grouped_gemm_amd as moe


class _Lib:
    """The real library, with a fixed clock rate."""

    def __init__(self, real):
        self._real = real

    def moe_tile_clock_hz(self):
        return 100e6

    def __getattr__(self, name):
        return getattr(self._real, name)


def _pack(kind, nnb, wg, n, band):
    return kind | (nnb << 2) | (wg << 8) | (n << 24) | (band << 40)


def test_records_decode(monkeypatch):
    real = moe.lib()
    monkeypatch.setattr(moe, "lib", lambda: _Lib(real))
    p = moe.make_problem(T=512, d=256, f=256, E_global=8, k=2, trace=True)
    lay = moe.workspace_layout(p)
    assert lay.tile_trace_capacity > 3
    ws = torch.zeros(lay.total, dtype=torch.uint8)
    v = moe.workspace_views(p, ws)
    base = 10_000_000_000
    recs = [(base + 500, base + 520, base + 4_520, base + 4_700, _pack(1, 4, 255, 3, 17)),
            (base, base + 1, base + 2, base + 3, _pack(2, 2, 0, 65535, (1 << 24) - 1)),
            (base + 100, base + 300, base + 900, base + 1000, _pack(2, 4, 65535, 0, 0))]
    arr = np.array(recs, dtype=np.uint64).view(np.int64)
    v["tile_trace"][:3] = torch.from_numpy(arr)
    v["meta"][4] = 3
    tr = moe.tile_trace(p, ws)
    np.testing.assert_array_equal(tr["kind"], [1, 2, 2])
    np.testing.assert_array_equal(tr["nnb"], [4, 2, 4])
    np.testing.assert_array_equal(tr["wg"], [255, 0, 65535])
    np.testing.assert_array_equal(tr["n"], [3, 65535, 0])
    np.testing.assert_array_equal(tr["band"], [17, (1 << 24) - 1, 0])
    # microseconds from the earliest start at 100 MHz
    np.testing.assert_allclose(tr["t_start"], [5.0, 0.0, 1.0])
    np.testing.assert_allclose(tr["t_end"], [47.0, 0.03, 10.0])
    np.testing.assert_allclose(tr["t_main_end"] - tr["t_ready"], [40.0, 0.01, 6.0])


def test_untraced_problem_has_no_region():
    p = moe.make_problem(T=512, d=256, f=256, E_global=8, k=2)
    lay = moe.workspace_layout(p)
    assert lay.tile_trace_capacity == 0
    ws = torch.zeros(lay.total, dtype=torch.uint8)
    assert "tile_trace" not in moe.workspace_views(p, ws)
