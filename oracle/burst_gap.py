"""The Burst–Gap model of store bursts, written out in float64.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the library, whose
calibration code (expert_grouped_gemm_amd/burst_gap.py) is written
separately. Pins: tests/test_oracle_burst_gap.py (the pages' worked capacity
figure, a discrete fluid-queue simulation of the text's assumptions).

Source: X-Stage (Xian et al.), Section 3 "Remote-Store Microbenchmarks" and
"The X-Stage Burst–Gap Model", Equations 1-7, and Section 4.1, the design
test of Equation 10. Notation as on that page (Table 1): K producers, B bytes
per producer per burst, aggregate volume V = K*B, producer-side gap G,
backpressure-free issue time T0 (T_iss^0), effective drain rate R, effective
outstanding capacity Q. Times in seconds, volumes in bytes, rates in bytes/s.
"""
from __future__ import annotations

import numpy as np


def pos(x):
    """[x]_+ = max(x, 0)."""
    return np.maximum(x, 0.0)


def t_iss(G, V, R, T0):
    """Sender-visible issue time of a periodic burst, Eq. 3: issue cannot be
    faster than the recovered floor T0; in the drain-limited regime a period
    (issue plus gap, Eq. 2) must last V / R (flow conservation, Eq. 1)."""
    return np.maximum(T0, V / R - G)


def t_period(G, V, R, T0):
    """Start-to-start period of periodic bursts: issue time plus gap (Eq. 2),
    with Eq. 3 substituted: max(T0 + G, V / R)."""
    return t_iss(G, V, R, T0) + G


def delta_t_iss(G, V, R, T0):
    """Backpressure overhead, Eq. 4: [V/R - G - T0]_+."""
    return pos(V / R - G - T0)


def g_star(V, R, T0):
    """Minimum recovery gap, Eq. 5: [V/R - T0]_+."""
    return pos(V / R - T0)


def q_peak(V, R, T0):
    """Peak outstanding volume of an isolated burst with no capacity limit,
    Eq. 6: what is injected during T0 minus what drains meanwhile."""
    return pos(V - R * T0)


def t_iss_isolated(V, R, T0, Q):
    """Issue time of one burst into an empty path, Eq. 7: injection beyond the
    capacity Q waits for the drain."""
    return np.maximum(T0, (V - Q) / R)


def design_test(V, G, R, T0, Q):
    """Eq. 10: no modeled backpressure when the long-term injection rate
    V / (T0 + G) stays within R and one burst's excess over what drains
    during its issue fits in Q. Returns (rate_ok, capacity_ok)."""
    return V / (T0 + G) <= R, pos(V - R * T0) <= Q
