"""Pins of the oracle's dispatch bookkeeping (readings R3-R5)."""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(__file__)


def test_dispatch_worked_example():
    with open(os.path.join(HERE, "golden", "dispatch_worked.json")) as fh:
        g = json.load(fh)
    idx = np.array(g["idx"], dtype=np.int32)
    w = np.array(g["w"])
    r = oracle.dispatch(idx, w, g["e_begin"], g["e_end"], g["S"])
    ex = g["expected"]
    for key in ("counts", "offsets", "row_src", "tok_off", "row_dst"):
        assert r[key].tolist() == ex[key], key
    np.testing.assert_array_equal(r["comb_w"], ex["comb_w"])
    assert np.bincount(idx.ravel(), minlength=g["E_global"]).tolist() == ex["counts_global"]


def _bruteforce_dispatch(idx, w, e_begin, e_end, S):
    """Pure-Python loops, a different construction from the oracle's."""
    T, k = idx.shape
    row_src = []
    counts = []
    for e in range(e_begin, e_end):
        n = 0
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    row_src.append(t * k + j)
                    n += 1
        counts.append(n)
    token_list = []
    tok_off = [0]
    for s in range(S):
        for t in range(s, T, S):
            for j in range(k):
                if e_begin <= idx[t, j] < e_end:
                    token_list.append(t * k + j)
            tok_off.append(len(token_list))
    row_dst = [token_list.index(a) for a in row_src]
    comb_w = [w[a // k, a % k] for a in token_list]
    return counts, row_src, row_dst, tok_off, comb_w


@pytest.mark.parametrize("T,E,k,eb,ee,S", [(16, 8, 2, 0, 8, 1), (24, 16, 4, 3, 9, 4), (32, 6, 3, 5, 6, 8),
                                           (8, 4, 4, 0, 4, 2), (40, 12, 1, 2, 7, 1)])
def test_dispatch_matches_bruteforce(T, E, k, eb, ee, S):
    rng = np.random.default_rng(T + E + k)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, w, counts_global = oracle.route_topk(L, k)
    r = oracle.dispatch(idx, w, eb, ee, S)
    counts, row_src, row_dst, tok_off, comb_w = _bruteforce_dispatch(idx, w, eb, ee, S)
    assert r["counts"].tolist() == counts
    assert r["row_src"].tolist() == row_src
    assert r["row_dst"].tolist() == row_dst
    assert r["tok_off"].tolist() == tok_off
    np.testing.assert_array_equal(r["comb_w"], comb_w)
    assert counts_global.sum() == T * k
    assert r["A"] == sum(counts) == r["offsets"][-1]


def test_dispatch_invariants_at_scale():
    rng = np.random.default_rng(0)
    T, E, k = 4096, 256, 8
    idx, w, cg = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    r = oracle.dispatch(idx, w, 0, 32, 8)
    A = r["A"]
    assert cg.sum() == T * k and r["counts"].sum() == A == cg[:32].sum()
    assert np.all(np.diff(r["offsets"]) >= 0) and np.all(r["counts"] <= T)
    rs = r["row_src"]
    e_of = idx.reshape(-1)[rs]
    assert np.all(np.diff(e_of) >= 0)                                  # expert-contiguous
    same = np.diff(e_of) == 0
    assert np.all(np.diff(rs)[same] > 0)                               # ascending a within expert
    assert sorted(r["row_dst"].tolist()) == list(range(A))            # a permutation
    assert np.all(r["tok_list"][r["row_dst"]] == rs)                   # row_dst inverts the token order
