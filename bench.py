#!/usr/bin/env python3
"""Benchmark of one GPU's share of the MoE layer on MI355X.

A step is one pass of the whole share (route -> dispatch -> grouped expert
GEMMs -> combine) over one batch of synthetic inputs already resident in HBM,
timed as one fused moe_layer_forward call per step, with nothing else on the
stream. Before the W warm-up steps, about 50 ms of untimed steps let the GPU
clock settle. After them, the same steps run again as the four component calls
(moe_route_topk, moe_dispatch, moe_expert_forward, moe_combine: the same
kernels) with HIP events between the stages on the launch stream, for the
per-stage times.
Then the expert-GEMM call runs alone, back to back between two events, for
the average launch duration that the roofline fraction divides by.

Default workload: the DeepSeek-style share (T=4096 tokens, d=7168, f=2048,
top-8 of 256 experts, this GPU owns experts 0-31, bf16). Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config NAME] [--sched auto|interleaved|expert_wave|separate]
                  [--no-cpu-baseline] [--no-compare] [--trace] [--copy-probe] [--owner-return TB_M]

After the main measurement the same steps are timed under each explicit
schedule (schedules_TFLOPs), unless --no-compare. --owner-return adds the
owner-aligned return path's stages (padded gather, GEMM on the padded layout,
segment copy, and for bf16 the overlapped copy) as an "owner_return" object.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5033.2    # MI355X dense fp8 MFMA
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the GPU reaches its steady clock after a few tens of ms of work")
    ap.add_argument("--config", default="deepseek_share_bf16")
    ap.add_argument("--sched", default="auto", choices=["auto", "interleaved", "expert_wave", "separate"],
                    help="expert-GEMM tile schedule (auto: the library's run-time choice)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip timing the other explicit schedules after the main measurement")
    ap.add_argument("--lead-D", type=int, default=0)
    ap.add_argument("--tiles", default="auto", choices=["auto", "narrow", "wide"],
                    help="expert-GEMM tile width (default: chosen from the shape)")
    ap.add_argument("--band-major", action="store_true", help="no grouped raster of the GEMM tile lists")
    ap.add_argument("--bf16-combine-buf", action="store_true",
                    help="MOE_FLAG_BF16_COMBINE_BUF: the token-ordered combine buffer in bf16 instead of fp32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace", action="store_true",
                    help="after the timed steps, run one call with per-tile timing and summarise the spans")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="tokens in the oracle's timed sample")
    ap.add_argument("--owner-return", type=int, default=0, metavar="TB_M",
                    help="also time the owner-aligned return path (8 owner ranks, this GPU rank 0, row bands of "
                         "TB_M rows, middle segments of 2 bands) after the timed steps")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also time a plain 1 GiB device copy (HBM reference and counter calibration)")
    return ap.parse_args()


def gemm_bytes(cfg, counts, cbuf_esz=4) -> float:
    """Algorithmic HBM bytes of one grouped-GEMM launch (Linear-1 + SwiGLU +
    Linear-2): each local expert with at least one row streams its W1 and W2
    once; per row: X row read (d), H write and read (2f), combine-buffer
    write (d elements of cbuf_esz bytes: 4, or 2 with the bf16 buffer)."""
    esz = 1 if cfg.dtype != "bf16" else 2              # activations (e4m3 for fp8 and W4A8)
    wesz = 0.5 + 1.0 / 32 if cfg.dtype == "w4a8_mxfp4" else esz   # MXFP4: 4-bit codes + an E8M0 byte per 32
    active = sum(1 for c in counts if c > 0)
    A = sum(counts)
    w = active * 3 * cfg.f * cfg.d * wesz
    rows = A * (cfg.d * esz + 2 * cfg.f * esz + cbuf_esz * cfg.d)
    return float(w + rows)


GEMM_SOURCES = ("gemm_device.h", "plan_device.h", "moe_internal.h", "gemm.hip", "gemm_bf16.hip", "gemm_fp8.hip", "gemm_w4a8.hip")


def gemm_source_digest():
    """First 16 hex digits of the SHA-256 of the expert-GEMM sources, in order."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "expert_grouped_gemm_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg, sched, tiles="auto", variant=False):
    """HBM bytes per grouped-GEMM launch measured with rocprofv3 FETCH_SIZE /
    WRITE_SIZE (scaled by a plain-copy calibration) for this workload and
    schedule, as recorded in profiles/gemm_traffic_<workload>_<sched>.md; null
    when no record exists, the GEMM source changed since it was taken, or the
    run is a variant the record does not cover (band-major order, bf16
    combine buffer)."""
    path = os.path.join(ROOT, "profiles", f"gemm_traffic_{cfg.name}_{sched}.md")
    if not os.path.exists(path):
        return None
    digest = gemm_source_digest()
    text = open(path).read()
    try:
        blob = json.loads(text.split("```json")[1].split("```")[0])
    except (IndexError, ValueError):
        return None
    if blob.get("gemm_source_sha256_16") != digest or blob.get("tiles", "auto") != tiles or variant:
        return None
    return blob.get("hbm_bytes_per_launch")


def trace_summary(moe, cfg, args, g, v):
    """One expert-GEMM call (outside the timed steps) with per-tile timing:
    per tile kind the mean readiness wait, K-loop and epilogue spans; the
    share of the workgroups' busy time spent in epilogues, which nothing in
    the same workgroup overlaps (the exposed stall of X-Stage Eq. 15 with an
    empty cover window); and how long workgroups sit idle at the end."""
    import numpy as np
    import torch
    p = moe.make_problem(cfg.T, cfg.d, cfg.f, cfg.E_global, cfg.k, cfg.e_begin, cfg.e_end, dtype=cfg.dtype,
                         num_segments=cfg.num_segments, sched=args.sched, lead_D=args.lead_D,
                         quant_block=cfg.quant_block, tiles=args.tiles, band_major=args.band_major, trace=True)
    ws = moe.alloc_workspace(p)
    # the dispatch outputs of the timed steps stand for this call's
    v2 = moe.workspace_views(p, ws)
    for key in ("offsets", "row_dst"):
        v2[key].copy_(v[key])
    moe.expert_forward(p, v["x_perm"], v.get("x_perm_scale"), v2["offsets"], v2["row_dst"], g["W1"],
                       g.get("W1_scale"), g["W2"], g.get("W2_scale"), v2["combine_buf"], ws)
    torch.cuda.synchronize()
    moe.check_workspace(p, ws)
    tr = moe.tile_trace(p, ws)
    t0, t1 = float(tr["t_start"].min()), float(tr["t_end"].max())
    span = t1 - t0
    busy = tr["t_end"] - tr["t_start"]
    wgs = np.unique(tr["wg"])
    last = np.array([tr["t_end"][tr["wg"] == w].max() for w in wgs])
    res = {"clock_hz": moe.lib().moe_tile_clock_hz(), "tiles": int(busy.size), "workgroups": int(wgs.size),
           "makespan_us": round(span, 2),
           "busy_frac": round(float(busy.sum()) / (wgs.size * span), 4),
           "epilogue_share": round(float((tr["t_end"] - tr["t_main_end"]).sum() / busy.sum()), 4),
           "tail_idle_us_mean": round(float((t1 - last).mean()), 2)}
    for k, name in ((1, "linear1"), (2, "linear2")):
        m = tr["kind"] == k
        res[name] = {"tiles": int(m.sum()),
                     "wait_us_mean": round(float((tr["t_ready"] - tr["t_start"])[m].mean()), 3),
                     "mainloop_us_mean": round(float((tr["t_main_end"] - tr["t_ready"])[m].mean()), 3),
                     "epilogue_us_mean": round(float((tr["t_end"] - tr["t_main_end"])[m].mean()), 3)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs one GPU's share of the layer; --gpus {args.gpus} is not supported on this "
              f"single-GPU build (the multi-GPU split is expert parallelism, documented, not run)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import expert_grouped_gemm_amd as moe
    import moe_synth

    cfg = moe_synth.CONFIGS[args.config]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    fp8 = cfg.dtype != "bf16"   # e4m3 activations: fp8 and W4A8 (MXFP4 weights)

    g = moe_synth.generate(cfg, device=dev)
    torch.cuda.synchronize()
    p = moe.make_problem(cfg.T, cfg.d, cfg.f, cfg.E_global, cfg.k, cfg.e_begin, cfg.e_end, dtype=cfg.dtype,
                         num_segments=cfg.num_segments, sched=args.sched, lead_D=args.lead_D,
                         quant_block=cfg.quant_block, tiles=args.tiles, band_major=args.band_major,
                         bf16_combine_buf=args.bf16_combine_buf)
    cbuf_esz = 2 if args.bf16_combine_buf else 4
    ws = moe.alloc_workspace(p)
    v = moe.workspace_views(p, ws)
    Y = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None, p=p):
        if ev is not None:
            ev[0].record(stream)
        moe.route_topk(p, g["logits"], v["topk_idx"], v["topk_w"], None, stream)
        if ev is not None:
            ev[1].record(stream)
        moe.dispatch(p, g["X"], g.get("X_scale"), v["topk_idx"], v["topk_w"], v["counts"], v["offsets"],
                     v["row_src"], v["row_dst"], v["tok_off"], v["comb_w"], v["x_perm"], v.get("x_perm_scale"),
                     ws, stream)
        if ev is not None:
            ev[2].record(stream)
        moe.expert_forward(p, v["x_perm"], v.get("x_perm_scale"), v["offsets"], v["row_dst"], g["W1"],
                           g.get("W1_scale"), g["W2"], g.get("W2_scale"), v["combine_buf"], ws, stream)
        if ev is not None:
            ev[3].record(stream)
        moe.combine(p, v["combine_buf"], v["tok_off"], v["comb_w"], Y, None, stream)
        if ev is not None:
            ev[4].record(stream)

    def fused_step(p=p):
        # moe_layer_forward: the same four stages in one library call
        moe.layer_forward(p, g["X"], g.get("X_scale"), g["logits"], g["W1"], g.get("W1_scale"), g["W2"],
                          g.get("W2_scale"), Y, None, ws, stream)

    # Setup, before the contract's warm-up steps: about 50 ms of untimed
    # steps, so that the GPU clock has settled even when --warmup is small
    # (three warm-up steps alone left the timed steps about 7% slow).
    t_ramp = time.perf_counter()
    while True:
        fused_step()
        torch.cuda.synchronize()
        if time.perf_counter() - t_ramp > 0.05:
            break
    for _ in range(args.warmup):
        fused_step()
    step()  # the component calls once, before their instrumented pass below
    torch.cuda.synchronize()
    moe.check_workspace(p, ws)

    # the timed steps: one fused layer call each, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fused_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    moe.check_workspace(p, ws)

    # Outside the timed steps, the same box: the four component calls back to
    # back (no events), the launch chain the fused call replaces.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    chain_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    moe.check_workspace(p, ws)

    # Outside the timed steps: the same steps with an event between stages for
    # the stage breakdown (each event record leaves the stream idle for a few
    # microseconds, so these steps run slower than the timed ones), then the
    # expert-GEMM call alone, back to back, for its average launch duration.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        moe.expert_forward(p, v["x_perm"], v.get("x_perm_scale"), v["offsets"], v["row_dst"], g["W1"],
                           g.get("W1_scale"), g["W2"], g.get("W2_scale"), v["combine_buf"], ws, stream)
    g1.record(stream)
    torch.cuda.synchronize()
    moe.check_workspace(p, ws)

    stage_proto = stage_protocol(moe, cfg, p, g, v, ws, Y, stream)

    stage_names = ["route", "dispatch", "expert_gemm", "combine"]
    per = {n: [events[i][j].elapsed_time(events[i][j + 1]) * 1e3 for i in range(args.steps)]
           for j, n in enumerate(stage_names)}
    med = {n: statistics.median(x) for n, x in per.items()}
    gemm_call_us = g0.elapsed_time(g1) * 1e3 / args.steps

    counts = v["counts"].cpu().tolist()
    A = int(sum(counts))
    ms_per_step = wall * 1e3 / args.steps
    useful_flop = 6.0 * A * cfg.d * cfg.f
    tflops = useful_flop / (ms_per_step * 1e-3) / 1e12
    peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS

    esz = 1 if fp8 else 2
    gb = gemm_bytes(cfg, counts, cbuf_esz)
    gemm_us = gemm_call_us
    # The grouped GEMM is bound by HBM when its arithmetic intensity (useful
    # FLOP per algorithmic byte) is below the ridge point peak_flops / 8 TB/s.
    intensity = useful_flop / gb
    ridge = peak * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if intensity < ridge:
        bound, achieved, rpeak, runit = "hbm", gb / (gemm_us * 1e-6) / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        bound, achieved, rpeak, runit = "mfma", useful_flop / (gemm_us * 1e-6) / 1e12, peak, "TFLOP/s"
    disp_bytes = 2.0 * A * cfg.d * esz + cfg.T * cfg.k * 8.0
    comb_bytes = A * cfg.d * float(cbuf_esz) + cfg.T * cfg.d * 2.0
    out = {
        "metric": "fused MoE-layer useful TFLOP/s (6*A*d*f per step); % of MFMA peak; dispatch/combine GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens and logits, N(0,0.02) weights, drawn on the GPU)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "f": cfg.f, "E_global": cfg.E_global,
                   "k": cfg.k, "local_experts": [cfg.e_begin, cfg.e_end], "segments": cfg.num_segments,
                   "sched": args.sched, "sched_run": moe.schedule_of(p), "tiles": args.tiles,
                   "band_major": args.band_major, "bf16_combine_buf": args.bf16_combine_buf,
                   "A_local_assignments": A, "parallelism": "single GPU (one EP share)"},
        "pct_mfma_peak": round(100.0 * tflops / peak, 2),
        "component_calls_ms_per_step": round(chain_ms, 4),
        "component_calls_note": "the same step as moe_route_topk, moe_dispatch, moe_expert_forward and moe_combine "
                                "back to back (the launch chain the fused moe_layer_forward replaces), same process",
        "stages_us_median": {n: round(x, 2) for n, x in med.items()},
        "stages_note": "from separate steps with an event between stages, after the timed steps",
        "dispatch_GBps": round(disp_bytes / (stage_proto["dispatch"]["median_us"] * 1e-6) / 1e9, 1),
        "combine_GBps": round(comb_bytes / (stage_proto["combine"]["median_us"] * 1e-6) / 1e9, 1),
        "dispatch_combine_protocol": dict(
            stage_proto,
            algorithmic_bytes={"dispatch": disp_bytes, "combine": comb_bytes},
            frac_of_hbm_peak={"dispatch": round(disp_bytes / (stage_proto["dispatch"]["median_us"] * 1e-6) / 1e9
                                                / HBM_PEAK_GBPS, 4),
                              "combine": round(comb_bytes / (stage_proto["combine"]["median_us"] * 1e-6) / 1e9
                                               / HBM_PEAK_GBPS, 4)},
            note="moe_dispatch and moe_combine each timed alone, 20 trials after one warm-up call, a 512 MiB "
                 "read before every trial evicting the 256 MiB last-level cache; copy_GBps is a device-to-device "
                 "copy of the combine's byte count under the same protocol (the achievable streaming rate)"),
        "roofline": {
            "kernel": "moe_gemm_kernel (grouped Linear-1+SwiGLU+Linear-2, one persistent launch)"
            if moe.schedule_of(p) != "separate" else "moe_gemm_kernel (Linear-1 launch + Linear-2 launch)",
            "bound": bound,
            "achieved": round(achieved, 1),
            "peak": rpeak,
            "unit": runit,
            "frac": round(achieved / rpeak, 4),
            "traffic": measured_traffic(cfg, moe.schedule_of(p), args.tiles, args.band_major or args.bf16_combine_buf),
            "algorithmic_bytes_per_launch": gb,
            "useful_flop_per_launch": useful_flop,
            "arithmetic_intensity_flop_per_byte": round(intensity, 1),
            "avg_launch_us": round(gemm_us, 2),
            "launches_per_call": 2 if moe.schedule_of(p) == "separate" else 1,
            "avg_launch_us_note": "one moe_expert_forward call: the planning kernel and the GEMM launch(es), "
                                  "timed back to back with HIP events on the launch stream",
        },
    }

    if not args.no_compare:
        # the same steps under each explicit schedule (same inputs and workspace)
        rates = {}
        for sname in ("separate", "interleaved", "expert_wave"):
            ps = moe.make_problem(cfg.T, cfg.d, cfg.f, cfg.E_global, cfg.k, cfg.e_begin, cfg.e_end,
                                  dtype=cfg.dtype, num_segments=cfg.num_segments, sched=sname,
                                  quant_block=cfg.quant_block, tiles=args.tiles, band_major=args.band_major)
            for _ in range(args.warmup):
                fused_step(p=ps)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                fused_step(p=ps)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / args.steps
            moe.check_workspace(ps, ws)
            rates[sname] = round(useful_flop / dt / 1e12, 2)
        out["schedules_TFLOPs"] = rates

    if args.trace:
        out["tile_trace"] = trace_summary(moe, cfg, args, g, v)

    if args.owner_return:
        out["owner_return"] = owner_return_summary(moe, cfg, args, g, v, gemm_call_us, A)

    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 10
        out["copy_probe"] = {"bytes_moved": 2 * n, "us": round(us, 2), "GBps": round(2 * n / (us * 1e-6) / 1e9, 1)}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, g, args)

    print(json.dumps(out), flush=True)


def owner_return_summary(moe, cfg, args, g, v, gemm_std_us, A):
    """Owner-aligned return path (Cui et al., Sections 3.2-3.3) on this
    workload: host plan from the routing in the workspace, padded gather,
    the grouped GEMM on the padded layout, segment copy into the receive
    buffer. Each device stage is timed back to back with HIP events."""
    import torch
    S, local, x, tb = 8, 0, 2, args.owner_return
    p8 = moe.make_problem(cfg.T, cfg.d, cfg.f, cfg.E_global, cfg.k, cfg.e_begin, cfg.e_end, dtype=cfg.dtype,
                          num_segments=S, sched="separate", quant_block=cfg.quant_block)
    plan = moe.owner_plan(p8, v["topk_idx"].cpu().numpy(), local, tb, x)
    R = plan["R"]
    p8.row_capacity = max(R, moe.row_capacity(p8))  # the workspace holds the padded rows
    res = {"owner_ranks": S, "local_rank": local, "tb_M": tb, "x_bands": x, "A": A, "R_padded": R,
           "padding_ratio": round(R / max(A, 1), 4), "bands": plan["n_bands"],
           "remote_bands": plan["remote_bands"], "segments": plan["n_segments"],
           "expert_gemm_us_unpadded": round(gemm_std_us, 2)}
    fp8 = cfg.dtype != "bf16"
    cap = moe.row_capacity(p8)
    stream = torch.cuda.current_stream()
    row_src = torch.from_numpy(plan["row_src"]).cuda()
    X_pad = torch.empty((R, cfg.d), dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
    X_pad_scale = torch.empty((cfg.d // 128, cap), dtype=torch.float32, device="cuda") if fp8 else None
    O_pad = torch.empty((R, cfg.d), dtype=torch.float32, device="cuda")
    eo = torch.from_numpy(plan["expert_off"]).cuda()
    iota = torch.arange(R, dtype=torch.int32, device="cuda")
    segs = torch.from_numpy(plan["segments"]).cuda().contiguous()
    recv = torch.empty((plan["recv_rows"], cfg.d), dtype=torch.float32, device="cuda")
    ws8 = moe.alloc_workspace(p8)
    stages = {
        "gather": lambda: moe.owner_gather(p8, g["X"], g.get("X_scale"), row_src, X_pad, X_pad_scale, stream),
        "expert_gemm": lambda: moe.expert_forward(p8, X_pad, X_pad_scale, eo, iota, g["W1"], g.get("W1_scale"),
                                                  g["W2"], g.get("W2_scale"), O_pad, ws8, stream),
        "segment_copy": lambda: moe.segment_copy(p8, O_pad, segs, recv, stream),
    }
    n = max(10, args.steps // 2)
    for name, fn in stages.items():
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / n, 2)
    moe.check_workspace(p8, ws8)
    res["gather_GBps"] = round((A + R) * cfg.d * (1 if fp8 else 2) / (res["gather_us"] * 1e-6) / 1e9, 1)
    res["segment_copy_GBps"] = round(2 * A * cfg.d * 4 / (res["segment_copy_us"] * 1e-6) / 1e9, 1)
    res["segment_copy_frac_hbm"] = round(res["segment_copy_GBps"] / HBM_PEAK_GBPS, 4)
    if fp8:
        res["overlap_note"] = ("not run: the fp8 GEMM's wavefronts take a SIMD's whole register file, so the "
                               "waiting copier cannot share a compute unit with it")
        return res
    # Overlap (Cui et al., Section 3.3): the signalling GEMM on the launch
    # stream and the waiting copier on a second stream, against the same two
    # stages run one after the other.
    side = torch.cuda.Stream()
    row_done = torch.zeros((R + 31) // 32, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev = torch.cuda.Event()

    # the signalling GEMM walks its tile lists band by band, so that bands
    # complete one after another while the Linear-2 launch runs
    p8b = moe.make_problem(cfg.T, cfg.d, cfg.f, cfg.E_global, cfg.k, cfg.e_begin, cfg.e_end, dtype=cfg.dtype,
                           num_segments=S, sched="separate", quant_block=cfg.quant_block, band_major=True,
                           row_capacity=p8.row_capacity)

    # Every variant clears row_done first, so that the four carry the same
    # extra work; the copier's error word is checked after each.
    def gemm_signal():
        row_done.zero_()
        moe.expert_forward_signal(p8b, X_pad, X_pad_scale, eo, iota, g["W1"], g.get("W1_scale"), g["W2"],
                                  g.get("W2_scale"), O_pad, row_done, ws8, stream)

    def overlapped():
        row_done.zero_()
        ev.record(stream)
        side.wait_event(ev)
        # the GEMM first: on a shared hardware queue the copier then follows it
        moe.expert_forward_signal(p8b, X_pad, X_pad_scale, eo, iota, g["W1"], g.get("W1_scale"), g["W2"],
                                  g.get("W2_scale"), O_pad, row_done, ws8, stream)
        moe.segment_copy_wait(p8, O_pad, R, segs, recv, row_done, err, 0, side)
        stream.wait_stream(side)

    def overlapped_raster():
        # the same pair with the GEMM's default (grouped raster) tile order
        row_done.zero_()
        ev.record(stream)
        side.wait_event(ev)
        moe.expert_forward_signal(p8, X_pad, X_pad_scale, eo, iota, g["W1"], g.get("W1_scale"), g["W2"],
                                  g.get("W2_scale"), O_pad, row_done, ws8, stream)
        moe.segment_copy_wait(p8, O_pad, R, segs, recv, row_done, err, 0, side)
        stream.wait_stream(side)

    def sequential():
        row_done.zero_()
        stages["expert_gemm"]()
        stages["segment_copy"]()

    for name, fn in (("expert_gemm_signal", gemm_signal), ("sequential", sequential), ("overlapped", overlapped),
                     ("overlapped_raster_order", overlapped_raster)):
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / n, 2)
        if int(err.item()) != 0:
            raise RuntimeError(f"moe_segment_copy_wait: a readiness wait timed out ({name})")
    moe.check_workspace(p8, ws8)
    res["overlap_ratio"] = round((res["sequential_us"] - res["overlapped_us"]) / res["segment_copy_us"], 3)
    res["overlap_note"] = ("overlap_ratio = (sequential - overlapped) / segment_copy: the share of the copy "
                           "hidden under the GEMM (the signalling GEMM's own cost included)")
    res["gather_GBps"] = round((A + R) * cfg.d * (1 if fp8 else 2) / (res["gather_us"] * 1e-6) / 1e9, 1)
    res["segment_copy_GBps"] = round(2 * A * cfg.d * 4 / (res["segment_copy_us"] * 1e-6) / 1e9, 1)
    res["segment_copy_frac_hbm"] = round(res["segment_copy_GBps"] / HBM_PEAK_GBPS, 4)
    return res


def stage_protocol(moe, cfg, p, g, v, ws, Y, stream, trials=20):
    """moe_dispatch and moe_combine timed standalone: one warm-up call, then
    `trials` trials each preceded by a 512 MiB read that evicts the 256 MiB
    last-level cache, HIP events on the launch stream around the call alone;
    median, p10 and p90 in microseconds. A device-to-device copy of the
    combine's algorithmic byte count (read + write) is timed the same way.
    The flush reads rather than writes: a written flush leaves up to 256 MiB
    of dirty lines whose write-back then lands inside the timed call (it
    slowed the same copy by about 45%)."""
    import numpy as np
    import torch
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    esz = 1 if cfg.dtype != "bf16" else 2
    A = int(v["offsets"][-1])
    comb_bytes = A * cfg.d * (2 if p.flags & moe.FLAG_BF16_COMBINE_BUF else 4) + cfg.T * cfg.d * 2
    half = comb_bytes // 2 // 16 * 16
    src = torch.empty(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    calls = {
        "dispatch": lambda: moe.dispatch(p, g["X"], g.get("X_scale"), v["topk_idx"], v["topk_w"], v["counts"],
                                         v["offsets"], v["row_src"], v["row_dst"], v["tok_off"], v["comb_w"],
                                         v["x_perm"], v.get("x_perm_scale"), ws, stream),
        "combine": lambda: moe.combine(p, v["combine_buf"], v["tok_off"], v["comb_w"], Y, None, stream),
        "copy": lambda: dst.copy_(src),
    }
    out = {}
    for name, fn in calls.items():
        fn()
        us = []
        for _ in range(trials):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3)
        a = np.array(us)
        out[name] = {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
                     "p90_us": round(float(np.percentile(a, 90)), 2)}
    out["copy_GBps"] = round(2 * half / (out["copy"]["median_us"] * 1e-6) / 1e9, 1)
    moe.check_workspace(p, ws)
    return out


def cpu_baseline(cfg, g, args):
    """The oracle (fp64 NumPy) as it stands, timed on this host on a bounded
    sample: routing and dispatch of all T tokens plus the expert FFNs and the
    combine of the first n tokens' local assignments, n doubling from 256
    until one run takes at least 10 s (or covers every token). Rate = useful
    FLOP of the sampled assignments / wall time of that run."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    host = {k: t.cpu() for k, t in g.items()}
    n = args.cpu_sample_tokens or 256
    while True:
        n = min(n, cfg.T)
        t0 = time.perf_counter()
        r = oracle.moe_layer(host, cfg, tokens=np.arange(n))
        dt = time.perf_counter() - t0
        if dt >= 10.0 or n >= cfg.T or args.cpu_sample_tokens:
            break
        n *= 2
    A_s = int(np.sum(r["row_src"] // cfg.k < n))
    flop = 6.0 * A_s * cfg.d * cfg.f
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{blas.get('name')} {blas.get('version')}"
    except Exception:
        blas = "unknown"
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": f"first {n} of {cfg.T} tokens ({A_s} local assignments; routing+dispatch of all tokens), "
                      f"{dt:.1f} s"}


if __name__ == "__main__":
    main()
