"""moe_dispatch_noalloc (the dispatch with library-owned scratch, for callers
that cannot allocate) against moe_dispatch with a workspace, through the C
ABI: every output bit-exact, on two calls in a row, the second with a
smaller input (the shared scratch keeps the first call's contents), then an
fp8 call; and a problem whose scratch exceeds the array is refused before
any launch."""
import ctypes

import pytest
import torch

import expert_grouped_gemm_amd as moe
import moe_synth
from moe_cases import problem_of, to_gpu

pytestmark = pytest.mark.gpu

CASES = [
    moe_synth.make_config("tiny", T=1000, d=384, f=384, E_global=16, k=4, e_begin=3, e_end=11, num_segments=4,
                          seed=41),
    moe_synth.make_config("tiny", T=256, d=256, f=256, E_global=16, k=2, e_begin=0, e_end=5, seed=42),
    moe_synth.make_config("tiny", T=384, d=256, f=256, E_global=32, k=4, e_begin=8, e_end=24, num_segments=8,
                          dtype="fp8_e4m3", seed=43),
]


def _outputs(cfg, p):
    El, cap = cfg.E_local, moe.row_capacity(p)
    fp8 = cfg.dtype == "fp8_e4m3"
    i32 = dict(dtype=torch.int32, device="cuda")
    return dict(counts=torch.full((El,), -1, **i32), offsets=torch.full((El + 1,), -1, **i32),
                row_src=torch.full((cap,), -1, **i32), row_dst=torch.full((cap,), -1, **i32),
                tok_off=torch.full((cfg.T + 1,), -1, **i32),
                comb_w=torch.full((cap,), -1.0, dtype=torch.float32, device="cuda"),
                X_perm=torch.zeros((cap, cfg.d), dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda"),
                X_perm_scale=torch.zeros((cfg.d // 128, cap), dtype=torch.float32, device="cuda") if fp8 else None)


def test_noalloc_dispatch_matches_workspace_dispatch():
    for i, cfg in enumerate(CASES):
        print(f"[no-alloc] call {i}: T={cfg.T} E_l={cfg.E_local} k={cfg.k} {cfg.dtype}", flush=True)
        g = to_gpu(moe_synth.generate(cfg))
        p = problem_of(cfg, sched="separate")
        idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
        moe.route_topk(p, g["logits"], idx, w)
        ws = moe.alloc_workspace(p)
        a, b = _outputs(cfg, p), _outputs(cfg, p)
        moe.dispatch(p, g["X"], g.get("X_scale"), idx, w, a["counts"], a["offsets"], a["row_src"], a["row_dst"],
                     a["tok_off"], a["comb_w"], a["X_perm"], a["X_perm_scale"], ws)
        moe.dispatch_noalloc(p, g["X"], g.get("X_scale"), idx, w, b["counts"], b["offsets"], b["row_src"],
                             b["row_dst"], b["tok_off"], b["comb_w"], b["X_perm"], b["X_perm_scale"])
        torch.cuda.synchronize()
        moe.check_workspace(p, ws)
        A = int(a["offsets"][-1])
        assert A > 0
        sl = dict(counts=slice(None), offsets=slice(None), tok_off=slice(None), row_src=slice(0, A),
                  row_dst=slice(0, A), comb_w=slice(0, A), X_perm=slice(0, A))
        for key, s in sl.items():
            x, y = a[key][s], b[key][s]
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            assert torch.equal(x, y), (i, key)
        if a["X_perm_scale"] is not None:
            assert torch.equal(a["X_perm_scale"][:, :A], b["X_perm_scale"][:, :A]), (i, "X_perm_scale")


def test_noalloc_refuses_problems_past_its_scratch():
    # 4M tokens: 16 MiB of per-row counts alone, beyond the 8 MiB array. The
    # pointers are never used: the size check comes before any launch.
    p = moe.make_problem(T=1 << 22, d=128, f=128, E_global=8, k=1, e_begin=0, e_end=2)
    fake = ctypes.c_void_p(1 << 20)
    st = moe.lib().moe_dispatch_noalloc(ctypes.byref(p), fake, None, fake, fake, fake, fake, fake, fake, fake, fake,
                                        fake, None, None)
    assert st == 2
