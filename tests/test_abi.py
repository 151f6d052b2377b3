"""The C-ABI library loads, exports every symbol include/moe_mi355x.h
declares, and validates arguments on the host (no GPU needed: every case here
is rejected before anything is enqueued)."""
import ctypes
import os
import re

import pytest

import expert_grouped_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from expert_grouped_gemm_amd import build
        build.build()
    return moe.lib()


def _declared():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", src)
    return sorted(set(names))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.moe_version().decode().count(".") == 2
    for s in range(6):
        assert L.moe_status_string(s)
    assert L.moe_status_string(99) == b"unknown status"


def test_struct_sizes_match_header():
    assert ctypes.sizeof(moe.Problem) == 16 * 4
    assert ctypes.sizeof(moe.WorkspaceLayout) == 18 * 8


GOOD = dict(T=64, d=128, f=256, E_global=4, k=2)


@pytest.mark.parametrize("over,code", [
    (dict(k=17, E_global=32), 2), (dict(k=5, E_global=4), 2), (dict(E_global=2048, k=2), 2),
    (dict(d=100), 2), (dict(f=192), 2), (dict(T=0), 2), (dict(e_begin=3, e_end=3), 2),
    (dict(e_begin=0, e_end=5), 2), (dict(num_segments=3), 2),
    # cap * d past 2^31 elements: the kernels' 32-bit row and byte offsets
    (dict(T=1 << 21, d=1024), 2),
])
def test_unsupported_shapes(L, over, code):
    kw = dict(GOOD)
    kw.update(over)
    p = moe.make_problem(**kw)
    assert L.moe_workspace_size(ctypes.byref(p)) == 0
    out = moe.WorkspaceLayout()
    assert L.moe_workspace_get_layout(ctypes.byref(p), ctypes.byref(out)) == code


def test_invalid_enums_and_flags(L):
    for field, val in (("dtype", 7), ("sched", 4), ("sched", -1), ("flags", 12), ("flags", 256), ("lead_D", -1),
                       ("grid", -2), ("row_capacity", -1)):
        p = moe.make_problem(**GOOD)
        setattr(p, field, val)
        out = moe.WorkspaceLayout()
        assert L.moe_workspace_get_layout(ctypes.byref(p), ctypes.byref(out)) == 1, field


def test_layout_is_aligned_and_disjoint(L):
    p = moe.make_problem(T=1000, d=384, f=384, E_global=16, k=4, e_begin=3, e_end=11, num_segments=4)
    lay = moe.workspace_layout(p)
    offs = [getattr(lay, n) for n, _ in moe.WorkspaceLayout._fields_ if n != "total"]
    assert all(o % 256 == 0 for o in offs)
    cap = 1000 * 4
    sizes = dict(topk_idx=4000 * 4, topk_w=4000 * 4, counts=8 * 4, offsets=9 * 4, row_src=cap * 4, row_dst=cap * 4,
                 tok_off=1001 * 4, comb_w=cap * 4, x_perm=cap * 384 * 2, h=cap * 384 * 2, combine_buf=cap * 384 * 4,
                 meta=64 * 4)
    spans = sorted((getattr(lay, n), getattr(lay, n) + s) for n, s in sizes.items())
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= lay.total == moe.workspace_size(p)


def test_null_and_small_workspace_rejected_before_launch(L):
    p = moe.make_problem(**GOOD)
    need = L.moe_workspace_size(ctypes.byref(p))
    fake = ctypes.c_void_p(1 << 20)           # never dereferenced: validation fails first
    none5 = [None] * 5                        # the optional routing / dispatch outputs

    def layer(*a, outs=none5):
        return L.moe_layer_forward(ctypes.byref(p), *a, *outs, None)
    # X NULL; then X_scale given for bf16 (inconsistent)
    assert layer(None, None, fake, fake, None, fake, None, fake, None, fake, ctypes.c_size_t(need)) == 1
    assert layer(fake, fake, *([fake] * 8), ctypes.c_size_t(need)) == 1
    # bf16 with a non-NULL W1 scale pointer is inconsistent
    assert layer(fake, None, fake, fake, fake, fake, None, fake, None, fake, ctypes.c_size_t(need)) == 1
    # workspace smaller than required
    assert layer(fake, None, fake, fake, None, fake, None, fake, None, fake, ctypes.c_size_t(need - 1)) == 3
    # misaligned workspace / tensors / optional outputs
    assert layer(fake, None, fake, fake, None, fake, None, fake, None, ctypes.c_void_p((1 << 20) + 16),
                 ctypes.c_size_t(need)) == 1
    assert layer(fake, None, fake, fake, None, fake, None, fake, None, fake, ctypes.c_size_t(need),
                 outs=[None, None, ctypes.c_void_p((1 << 20) + 2), None, None]) == 1
    # MOE_FLAG_FP32_Y_DEBUG without a Y_fp32 buffer
    p.flags = moe.FLAG_FP32_Y_DEBUG
    assert layer(fake, None, fake, fake, None, fake, None, fake, None, fake, ctypes.c_size_t(need)) == 1
    p.flags = 0
    assert L.moe_combine(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 4), fake, fake, fake, None, None) == 1
    assert L.moe_route_topk(ctypes.byref(p), None, fake, fake, None, None) == 1
    assert L.moe_route_topk(None, fake, fake, fake, None, None) == 1


def test_row_capacity_sizes_the_workspace(L):
    """row_capacity raises the rows the GEMM regions hold (a padded layout),
    never lowers them below T * min(k, E_l)."""
    base = moe.make_problem(T=256, d=128, f=256, E_global=8, k=2, e_begin=0, e_end=4)
    small = moe.make_problem(T=256, d=128, f=256, E_global=8, k=2, e_begin=0, e_end=4, row_capacity=100)
    big = moe.make_problem(T=256, d=128, f=256, E_global=8, k=2, e_begin=0, e_end=4, row_capacity=2000)
    assert moe.workspace_size(small) == moe.workspace_size(base)
    lb, lg = moe.workspace_layout(base), moe.workspace_layout(big)
    assert moe.row_capacity(big) == 2000 and moe.row_capacity(base) == 512
    assert lg.combine_buf - lg.h >= 2000 * 256 * 2
    assert lg.total - lb.total >= (2000 - 512) * (128 * 2 + 256 * 2 + 128 * 4)


def test_bf16_combine_buffer_halves_its_region(L):
    p32 = moe.make_problem(**GOOD)
    p16 = moe.make_problem(**GOOD, bf16_combine_buf=True)
    cap = 64 * 2
    assert moe.workspace_size(p32) - moe.workspace_size(p16) >= cap * 128 * 2 - 256


def test_binding_rejects_cpu_tensors():
    import torch
    p = moe.make_problem(**GOOD)
    with pytest.raises(ValueError):
        moe.route_topk(p, torch.zeros(64, 4), torch.zeros(64, 2, dtype=torch.int32), torch.zeros(64, 2))


def test_schedule_of_resolves_auto(L):
    for name, code in moe.SCHED.items():
        p = moe.make_problem(**GOOD, sched=name)
        assert L.moe_schedule_of(ctypes.byref(p)) == (moe.SCHED["separate"] if name == "auto" else code)
    assert moe.schedule_of(moe.make_problem(**GOOD, sched="auto")) == "separate"
    p = moe.make_problem(**GOOD)
    p.sched = 4
    assert L.moe_schedule_of(ctypes.byref(p)) == -1
    assert L.moe_schedule_of(None) == -1


def test_store_burst_probe_rejects_bad_arguments(L):
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: validation fails first
    ok = dict(K=4, B=4096, reps=3, gap=1.0, buf_bytes=4 * 8192, rec_bytes=(2 * 4 * 3 + 1) * 8)

    def call(**over):
        a = dict(ok)
        a.update(over)
        return L.moe_store_burst_probe(a["K"], a["B"], a["reps"], ctypes.c_double(a["gap"]), fake,
                                       ctypes.c_size_t(a["buf_bytes"]), fake, ctypes.c_size_t(a["rec_bytes"]),
                                       None)
    for over in (dict(K=0), dict(K=5000), dict(B=1000), dict(B=0), dict(reps=0), dict(gap=-1.0),
                 dict(gap=float("nan")), dict(gap=2e5), dict(gap=1e5, reps=21), dict(buf_bytes=4 * 4096 - 1), dict(rec_bytes=24 * 8)):
        assert call(**over) == 1, over
    assert L.moe_store_burst_probe(4, 4096, 3, ctypes.c_double(1.0), None, ctypes.c_size_t(1 << 20), fake,
                                   ctypes.c_size_t(1 << 20), None) == 1


def test_binding_argument_counts_match_the_header(L):
    # Every declared entry point the binding describes takes as many
    # arguments in its ctypes signature as the header declares.
    src = ""
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src += open(os.path.join(ROOT, "include", fn)).read()
    decls = re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(([^;]*?)\)\s*;", src, flags=re.S)
    assert decls
    checked = 0
    for name, params in decls:
        params = params.strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        argtypes = getattr(L, name).argtypes
        if argtypes is None:
            continue
        assert len(argtypes) == n, (name, len(argtypes), n)
        checked += 1
    assert checked >= 15
