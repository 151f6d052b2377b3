"""Pins of the Burst–Gap model oracle (X-Stage, Section 3, Eqs. 1-7, 10).

* The page's worked capacity figure (tests/golden/burst_gap_worked.json).
* A discrete simulation of the fluid process the text assumes (injection no
  faster than the backpressure-free rate V / T0, blocked while the
  outstanding volume is at capacity Q; a work-conserving drain at rate R):
  its steady-state issue time and period, and its isolated-burst issue time,
  must match Eqs. 2, 3 and 7.
* Eq. 10's rate bound holds exactly when Eq. 4's overhead is zero.
"""
import json
import os

import numpy as np
import pytest

from oracle import burst_gap as bg

HERE = os.path.dirname(os.path.abspath(__file__))
MiB = 1024.0 * 1024.0


def test_pages_capacity_figure():
    g = json.load(open(os.path.join(HERE, "golden", "burst_gap_worked.json")))
    V = g["K"] * g["B_knee_bytes"]
    assert abs(V / MiB - g["V_knee_MiB"]) < g["tol_MiB"]
    Q = bg.q_peak(V, g["R_Bps"], g["T0_s"])
    assert abs(Q / MiB - g["Q_MiB"]) < g["tol_MiB"]
    # at the knee the isolated issue time is still on its floor, and just above it is not
    assert bg.t_iss_isolated(V, g["R_Bps"], g["T0_s"], Q) == pytest.approx(g["T0_s"])
    assert bg.t_iss_isolated(2 * V, g["R_Bps"], g["T0_s"], Q) > g["T0_s"]


def simulate(V, G, R, T0, Q, periods, dt):
    """Outstanding volume q; each burst injects V at rate V/T0 while q < Q
    (at q = Q injection can only follow the drain), then idles G; the drain
    removes R per unit time whenever q > 0. Returns the issue time and the
    start-to-start period of the last burst."""
    q = 0.0
    t = 0.0
    starts, issues = [], []
    for _ in range(periods):
        starts.append(t)
        left = V
        while left > 1e-9:
            room = Q - q + R * dt                  # what fits after this step's drain
            inj = min(left, V / T0 * dt, max(room, 0.0))
            q = max(q + inj - R * dt, 0.0)
            left -= inj
            t += dt
        issues.append(t - starts[-1])
        steps = int(round(G / dt))
        for _ in range(steps):
            q = max(q - R * dt, 0.0)
            t += dt
    return issues[-1], starts[-1] - starts[-2]


@pytest.mark.parametrize("G_over_gstar", [0.0, 0.3, 0.7, 1.3, 2.0])
def test_periodic_bursts_match_eqs_2_3(G_over_gstar):
    R, T0 = 1.0, 1.0               # units: volume per time, time
    V = 3.0                        # V / R = 3 > T0: drain-limited at small gaps
    Q = 5.0                        # Q > V: an isolated burst never binds; R * G < Q below
    gs = bg.g_star(V, R, T0)
    assert gs == pytest.approx(2.0)
    G = G_over_gstar * gs
    ti, tp = simulate(V, G, R, T0, Q, periods=40, dt=1e-3)
    assert ti == pytest.approx(float(bg.t_iss(G, V, R, T0)), abs=0.02)
    assert tp == pytest.approx(float(bg.t_period(G, V, R, T0)), abs=0.02)
    assert ti - T0 == pytest.approx(float(bg.delta_t_iss(G, V, R, T0)), abs=0.02)


@pytest.mark.parametrize("V", [0.5, 1.5, 3.0, 6.0])
def test_isolated_burst_matches_eq_7(V):
    R, T0, Q = 1.0, 1.0, 1.0
    ti, _ = simulate(V, 100.0, R, T0, Q, periods=2, dt=1e-3)
    # with the floor of Eq. 7 and the capacity knee of Eq. 6
    assert ti == pytest.approx(float(bg.t_iss_isolated(V, R, T0, Q)), abs=0.02)
    assert (bg.q_peak(V, R, T0) <= Q) == (ti <= T0 + 0.02)


def test_rate_bound_is_zero_overhead():
    rng = np.random.default_rng(3)
    for _ in range(200):
        V, G, R, T0 = rng.uniform(0.1, 10.0, 4)
        rate_ok, _ = bg.design_test(V, G, R, T0, Q=1e9)
        assert rate_ok == (bg.delta_t_iss(G, V, R, T0) == 0.0)
