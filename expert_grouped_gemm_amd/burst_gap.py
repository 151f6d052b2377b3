"""Burst–Gap calibration of CU-issued store bursts into local HBM.

The local-memory control of X-Stage, Section 3 ("Remote-Store
Microbenchmarks", "The X-Stage Burst–Gap Model", Sections 3.3-3.5), run on
this GPU with moe_store_burst_probe:

* drain rate R: zero-gap periodic bursts settle at a period of V / R
  (Eq. 1); R is the least-squares slope of V against the steady periods of
  the drain-dominated points, those whose zero-gap period clearly exceeds
  the same burst's issue time after a long gap (Section 3.3);
* backpressure-free issue time T0(K, V): the issue time after a long gap
  (Section 3.4);
* the gap sweep at one (K, V) against Eq. 3, T_iss = max(T0, V/R - G), with no
  parameter refitted (Section 3.4);
* effective capacity Q(K): isolated bursts (each after a long gap); above
  the knee T_iss = (V - Q) / R (Eq. 7), so each such point gives
  Q = V - R T_iss (Section 3.5).

Run ``python -m expert_grouped_gemm_amd.burst_gap [--out FILE]`` on a GPU for
a JSON summary. The fitting functions take plain arrays (seconds, bytes) and
need no GPU.
"""
from __future__ import annotations

import argparse
import json
import sys
from typing import Dict, List, Sequence

import numpy as np


# ----------------------------------------------------------------- fitting ---

def fit_drain_rate(volumes: Sequence[float], periods: Sequence[float]) -> float:
    """R minimising sum (T_i - V_i / R)^2 over points on the drain-limited
    plateau T_period = V / R: with x = 1/R, x = sum(V T) / sum(V^2)."""
    V = np.asarray(volumes, float)
    T = np.asarray(periods, float)
    return float((V * V).sum() / (V * T).sum())


def predicted_issue_time(G, V, R, T0):
    """Eq. 3 of the model (issue no faster than the recovered floor, a period
    no shorter than V / R)."""
    return np.maximum(T0, V / R - np.asarray(G, float))


def fit_capacity(volumes: Sequence[float], issue_times: Sequence[float], R: float,
                 frac: float = 0.7) -> float:
    """Q from isolated bursts of one producer count K at several volumes.
    Below the knee a burst issues at the backpressure-free injection rate
    (V / T0 roughly constant, the fastest rate seen); above it T_iss =
    (V - Q) / R (Eq. 7), so each point whose injection rate V / T_iss fell
    below `frac` of the fastest gives V - R T_iss. Returns their median, or
    NaN when no burst reached the capacity."""
    V = np.asarray(volumes, float)
    T = np.asarray(issue_times, float)
    rate = V / T
    sel = rate < frac * rate.max()
    if not sel.any():
        return float("nan")
    return float(np.median(V[sel] - R * T[sel]))


# ------------------------------------------------------------- measurement ---

def run_probe(K: int, B: int, reps: int, gap_us: float, buf, rec) -> Dict[str, np.ndarray]:
    """One probe launch; per producer and burst the issue time and the
    start-to-start period, in seconds."""
    import torch

    import expert_grouped_gemm_amd as moe
    print(f"  probe K={K} B={B} reps={reps} gap_us={gap_us}", flush=True)
    moe.store_burst_probe(K, B, reps, gap_us, buf, rec)
    torch.cuda.synchronize()
    hz = moe.lib().moe_tile_clock_hz()
    r = rec[:2 * K * reps].cpu().numpy().view(np.uint64).reshape(K, reps, 2).astype(np.int64)
    t_iss = (r[:, :, 1] - r[:, :, 0]) / hz
    t_period = np.diff(r[:, :, 0], axis=1) / hz
    return {"t_iss": t_iss, "t_period": t_period}


def steady(x: np.ndarray, skip: float = 0.25) -> float:
    """Median over producers and over the bursts after the first `skip`
    fraction (the path fills during those)."""
    n = x.shape[1]
    return float(np.median(x[:, int(n * skip):]))


def calibrate(K_list=(64, 256), B_zero=(64 << 10, 256 << 10, 1 << 20), reps: int = 48,
              B_iso=(4 << 10, 16 << 10, 32 << 10, 64 << 10, 128 << 10, 256 << 10, 1 << 20, 4 << 20),
              iso_reps: int = 6, iso_gap_us: float = 200.0, B_sweep: int = 64 << 10,
              gap_sweep_us=(0.0, 0.5, 1.0, 2.0, 3.0, 4.0, 6.0, 8.0, 16.0), min_drain_volume: float = 16 * 2**20,
              log=print) -> Dict:
    import torch

    import expert_grouped_gemm_amd as moe
    dev = torch.device("cuda")
    Kmax = max(K_list)
    ring = 2 * max(max(B_zero), max(B_iso), B_sweep)
    buf = torch.empty(Kmax * ring, dtype=torch.uint8, device=dev)
    rec = torch.zeros(2 * Kmax * max(reps, iso_reps) + 1, dtype=torch.int64, device=dev)

    # (1) zero-gap periodic bursts: the steady period per (K, V); R from the
    # large volumes, which settle on V / R (Section 3.3)
    # A point is drain-dominated when its zero-gap period clearly exceeds the
    # issue time of the same burst after a long gap; otherwise the producers'
    # own issue rate, not the drain, sets the period (few producers).
    zero = []
    for K in K_list:
        for B in B_zero:
            m = run_probe(K, B, reps, 0.0, buf[:K * ring], rec)
            z = {"K": K, "B": B, "V": K * B, "t_period": steady(m["t_period"]), "t_iss": steady(m["t_iss"])}
            mi = run_probe(K, B, iso_reps, iso_gap_us, buf[:K * ring], rec)
            z["t_iss_long_gap"] = steady(mi["t_iss"], skip=0.34)
            z["rate_Bps"] = z["V"] / z["t_period"]
            z["drain_dominated"] = z["t_period"] > 1.2 * z["t_iss_long_gap"]
            zero.append(z)
            log(f"zero gap  K={K:4d} B={B >> 10:5d} KiB: period {z['t_period'] * 1e6:8.2f} us "
                f"({z['rate_Bps'] / 1e9:7.1f} GB/s), long-gap issue {z['t_iss_long_gap'] * 1e6:8.2f} us"
                f"{', drain-dominated' if z['drain_dominated'] else ''}")
    dd = [z for z in zero if z["drain_dominated"]]
    if not dd:
        dd = [z for z in zero if z["V"] >= min_drain_volume]
    R = fit_drain_rate([z["V"] for z in dd], [z["t_period"] for z in dd])
    log(f"R = {R / 1e9:.1f} GB/s from {len(dd)} zero-gap points")

    # (2) isolated bursts at K = Kmax: the floor and the capacity knee (Section 3.5)
    iso = []
    for B in B_iso:
        m = run_probe(Kmax, B, iso_reps, iso_gap_us, buf[:Kmax * ring], rec)
        p = {"B": B, "V": Kmax * B, "t_iss": steady(m["t_iss"], skip=0.34)}
        iso.append(p)
        log(f"isolated  K={Kmax:4d} B={B >> 10:5d} KiB: issue {p['t_iss'] * 1e6:8.2f} us")
    Q = fit_capacity([p["V"] for p in iso], [p["t_iss"] for p in iso], R)
    # without a knee, Eq. 6 at the largest burst bounds Q from below
    Q_low = max(max(p["V"] - R * p["t_iss"], 0.0) for p in iso)
    log(f"Q = {Q / 2**20:.2f} MiB" if Q == Q else
        f"Q: no isolated burst reached the capacity; Q >= {Q_low / 2**20:.1f} MiB (Eq. 6 at the largest)")

    # (3) gap sweep at one (K, V) against Eq. 3 with R from (1) and T0 the
    # long-gap plateau of the same burst (Section 3.4): nothing refitted
    T0 = next(p["t_iss"] for p in iso if p["B"] == B_sweep)
    V = Kmax * B_sweep
    sweep = []
    for G in gap_sweep_us:
        m = run_probe(Kmax, B_sweep, reps, G, buf[:Kmax * ring], rec)
        ti = steady(m["t_iss"])
        pred = float(predicted_issue_time(G * 1e-6, V, R, T0))
        sweep.append({"G_us": G, "t_iss": ti, "predicted": pred, "t_period": steady(m["t_period"])})
        log(f"gap {G:5.1f} us: issue {ti * 1e6:7.3f} us, Eq. 3 {pred * 1e6:7.3f} us, "
            f"period {sweep[-1]['t_period'] * 1e6:7.3f} us")
    err = [abs(s["t_iss"] - s["predicted"]) / s["predicted"] for s in sweep]

    return {"clock_hz": moe.lib().moe_tile_clock_hz(), "R_Bps": R, "Q_bytes": Q, "Q_lower_bound_bytes": Q_low,
            "zero_gap": zero,
            "isolated": {"K": Kmax, "points": iso},
            "gap_sweep": {"K": Kmax, "B": B_sweep, "V": V, "T0_s": T0, "G_star_s": max(V / R - T0, 0.0),
                          "points": sweep, "median_rel_err_eq3": float(np.median(err)),
                          "max_rel_err_eq3": float(max(err))}}


def main(argv: List[str] = None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default=None, help="write the JSON summary here")
    a = ap.parse_args(argv)
    res = calibrate(log=lambda s: print(s, flush=True))
    text = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
