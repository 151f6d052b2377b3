"""Pins of the oracle's router (reading R1) against worked values and invariants."""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle

HERE = os.path.dirname(__file__)


def _golden():
    with open(os.path.join(HERE, "golden", "route_worked.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _golden())
def test_route_worked_examples(case):
    L = np.array([case["logits"]], dtype=np.float32)
    idx, w, counts = oracle.route_topk(L, case["k"])
    assert idx[0].tolist() == case["idx"]
    if case["w"] is not None:
        np.testing.assert_allclose(w[0], case["w"], rtol=0, atol=case["w_tol"])
    else:  # k = E: full softmax in slot order
        ref = scipy.special.softmax(L[0].astype(np.float64))[np.array(case["idx"])]
        np.testing.assert_allclose(w[0], ref, rtol=1e-13)
    assert counts.sum() == case["k"]


@pytest.mark.parametrize("T,E,k", [(257, 64, 4), (64, 256, 8), (33, 8, 2), (16, 1024, 16)])
def test_route_invariants(T, E, k):
    rng = np.random.default_rng(T * E + k)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[::5, :3] = L[::5, 3:4]            # constructed ties
    idx, w, counts = oracle.route_topk(L, k)
    assert counts.sum() == T * k                              # sum of counts = T*k
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    for t in range(T):
        sel = idx[t]
        assert len(set(sel.tolist())) == k                    # distinct
        unsel = np.setdiff1d(np.arange(E), sel)
        assert L[t, sel].min() >= (L[t, unsel].max() if unsel.size else -np.inf)
        v = L[t, sel]
        for j in range(k - 1):                                # slot order
            assert v[j] > v[j + 1] or (v[j] == v[j + 1] and sel[j] < sel[j + 1])
        # boundary ties resolved toward lower indices
        if unsel.size:
            tied_out = unsel[L[t, unsel] == v[-1]]
            assert np.all(tied_out > sel[v == v[-1]].max())
        assert abs(w[t].sum() - 1.0) < 1e-12
        assert np.all(np.diff(w[t]) <= 0)


def test_route_full_k_is_softmax():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((20, 12)).astype(np.float32)
    idx, w, _ = oracle.route_topk(L, 12)
    full = scipy.special.softmax(L.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, idx.astype(np.int64), axis=1), rtol=1e-12)


def test_route_bruteforce_subsets():
    """Tiny brute force: the selected set maximises the sum of logits among all
    k-subsets (ties aside), and equals a full descending sort's first k."""
    import itertools
    rng = np.random.default_rng(9)
    for _ in range(50):
        L = rng.standard_normal((1, 7)).astype(np.float32)
        idx, _, _ = oracle.route_topk(L, 3)
        best = max(itertools.combinations(range(7), 3), key=lambda s: sum(float(L[0, i]) for i in s))
        assert set(idx[0].tolist()) == set(best)
        assert idx[0].tolist() == sorted(best, key=lambda i: -float(L[0, i]))
