"""The store-burst probe (moe_store_burst_probe) on the GPU: every store
lands where the header says, and the clock readings are consistent with the
requested gap (the Burst–Gap microbenchmark of X-Stage, Section 3.1, in its
local-memory form)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,B,reps,gap_us", [(8, 16 << 10, 10, 2.0), (64, 4 << 10, 5, 0.0), (3, 1 << 10, 7, 0.5)])
def test_probe_stores_and_clock(K, B, reps, gap_us):
    import expert_grouped_gemm_amd as moe
    ring = 3 * B                                  # wraps after three bursts
    buf = torch.zeros(K * ring + 512, dtype=torch.uint8, device="cuda")
    rec = torch.zeros(2 * K * reps + 1, dtype=torch.int64, device="cuda")
    moe.store_burst_probe(K, B, reps, gap_us, buf[:K * ring], rec)
    torch.cuda.synchronize()
    hz = moe.lib().moe_tile_clock_hz()
    r = rec.cpu().numpy().view(np.uint64)
    assert r[-1] > 0                              # the common start time was published
    ts, ti = r[:-1].reshape(K, reps, 2)[:, :, 0].astype(np.int64), r[:-1].reshape(K, reps, 2)[:, :, 1].astype(np.int64)
    assert np.all(ti >= ts)
    period = np.diff(ts, axis=1) / hz
    # a period is at least the issue time plus the gap (one clock tick of slack)
    assert np.all(period >= (ti[:, :-1] - ts[:, :-1]) / hz + gap_us * 1e-6 - 2.0 / hz)
    # contents: the last burst written at each ring slot holds (burst, instruction, producer, lane)
    words = buf[:K * ring].cpu().numpy().view(np.uint32).reshape(K, ring // 1024, 64, 4)
    slots = ring // B
    per = B // 1024
    for k in range(K):
        for slot in range(slots):
            last = max(rr for rr in range(reps) if rr % slots == slot) if any(rr % slots == slot for rr in range(reps)) else None
            if last is None:
                continue
            blk = words[k, slot * per:(slot + 1) * per]
            want_i = np.arange(per)[:, None].repeat(64, 1)
            assert np.all(blk[:, :, 0] == last) and np.all(blk[:, :, 1] == want_i)
            assert np.all(blk[:, :, 2] == k) and np.all(blk[:, :, 3] == np.arange(64)[None, :])
    # nothing past the producers' rings was touched
    assert int(buf[K * ring:].sum()) == 0
