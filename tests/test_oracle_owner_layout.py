"""Pins of the owner-aligned return-path oracle (Cui et al., Sections 3.2,
3.3.2 and 4.5): a hand-worked example, the layout's defining properties on
random routings, the padding bound and the case that attains it, the segment
composition and two independent constructions of the receive buffer."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import owner_layout as ol

HERE = os.path.dirname(__file__)


def _route(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx, _, _ = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    return idx


def test_worked_example():
    with open(os.path.join(HERE, "golden", "owner_layout_worked.json")) as fh:
        g = json.load(fh)
    lay = ol.owner_aligned_layout(np.array(g["idx"]), g["e_begin"], g["e_end"], g["S"], g["local"], g["tb_M"])
    ex = g["expected"]
    for key in ("row_src", "expert_off", "band_expert", "band_dest", "band_row", "band_valid", "band_recv_off",
                "recv_rows", "recv_start"):
        assert lay[key].tolist() == ex[key], key
    assert ol.remote_first_schedule(lay).tolist() == ex["schedule"]


CASES = [(40, 8, 2, 0, 4, 4, 0, 4), (64, 16, 4, 4, 10, 8, 3, 8), (96, 6, 3, 1, 6, 3, 2, 5), (33, 4, 4, 0, 4, 2, 1, 1),
         (128, 32, 8, 0, 8, 8, 0, 32)]


@pytest.mark.parametrize("T,E,k,eb,ee,S,local,tb", CASES)
def test_layout_properties(T, E, k, eb, ee, S, local, tb):
    idx = _route(T, E, k, T + E)
    lay = ol.owner_aligned_layout(idx, eb, ee, S, local, tb)
    flat = idx.reshape(-1)
    rs = lay["row_src"]
    valid = rs[rs >= 0]
    # a permutation of the local assignments, plus zero rows
    expect = np.nonzero((flat >= eb) & (flat < ee))[0]
    assert sorted(valid.tolist()) == expect.tolist()
    rank_pos = {r: i for i, r in enumerate([r for r in range(S) if r != local] + [local])}
    off = lay["expert_off"]
    El = ee - eb
    for el in range(El):
        rows = rs[off[el]:off[el + 1]]
        v = rows[rows >= 0]
        assert np.all(flat[v] == eb + el)                                   # rows of this expert only
        key = [rank_pos[(a // k) % S] for a in v]
        assert key == sorted(key)                                           # remote ranks ascending, own last
        for r in range(S):
            g = [a for a in v if (a // k) % S == r]
            assert g == sorted(g)                                           # ascending assignment id
            n = len(g)
            assert lay["group_rows"][el, r] == n
            start = lay["group_off"][el, r] - off[el]
            assert start % tb == 0                                          # every group starts on a band
            grp = rows[start:start + (n if r == local else -(-n // tb) * tb)]
            assert grp[:n].tolist() == g and np.all(grp[n:] == -1)          # padding only at a group's end
        pad = int(np.sum(rows < 0))
        assert pad <= (S - 1) * (tb - 1)                                    # Section 4.5, per expert (L6)
    # every band has one owner; its valid rows lead; the band table covers the layout
    covered = np.zeros(len(rs), dtype=int)
    for b in range(len(lay["band_row"])):
        r0, nv, dst = lay["band_row"][b], lay["band_valid"][b], lay["band_dest"][b]
        height = min(tb, off[lay["band_expert"][b] + 1] - r0)
        covered[r0:r0 + height] += 1
        band = rs[r0:r0 + height]
        assert np.all(band[:nv] >= 0) and np.all(band[nv:] == -1)
        assert np.all((band[:nv] // k) % S == dst)
    assert np.all(covered == 1)
    assert lay["recv_rows"].sum() == len(valid)


def test_padding_bound_is_attained():
    # Section 4.5: (W-1)(tb_M-1) padded rows, 765 for W = 4 ranks and tb_M = 256.
    # One local expert; every remote rank sends 257 rows (one past a band).
    W, tb = 4, 256
    T = W * 257
    idx = np.zeros((T, 1), dtype=np.int32)
    lay = ol.owner_aligned_layout(idx, 0, 1, W, 0, tb)
    assert int(np.sum(lay["row_src"] < 0)) == (W - 1) * (tb - 1) == 765


@pytest.mark.parametrize("n,x,expect", [(1, 2, [1]), (2, 2, [1, 1]), (3, 2, [1, 1, 1]), (4, 2, [1, 2, 1]),
                                        (5, 2, [1, 2, 1, 1]), (6, 2, [1, 2, 2, 1]), (6, 3, [1, 3, 1, 1]),
                                        (5, 1, [1, 1, 1, 1, 1])])
def test_segment_composition(n, x, expect):
    # Figure 3b: first and last segment one band, middle segments x bands.
    tb = 4
    T = 2 * n * tb                          # rank 1 owns odd tokens: n full bands for expert 0
    idx = np.zeros((T, 1), dtype=np.int32)
    lay = ol.owner_aligned_layout(idx, 0, 1, 2, 0, tb)
    seg = ol.transfer_segments(lay, x)
    remote = seg["remote"] == 1
    assert seg["n_bands"][remote].tolist() == expect
    assert seg["rows"][remote].sum() == n * tb


@pytest.mark.parametrize("T,E,k,eb,ee,S,local,tb", CASES)
def test_schedule_and_segments_cover_once(T, E, k, eb, ee, S, local, tb):
    idx = _route(T, E, k, 7 * T + E)
    lay = ol.owner_aligned_layout(idx, eb, ee, S, local, tb)
    sched = ol.remote_first_schedule(lay)
    nb = len(lay["band_row"])
    assert sorted(sched.tolist()) == list(range(nb))
    is_remote = lay["band_dest"][sched] != local
    n_remote = int(is_remote.sum())
    assert np.all(is_remote[:n_remote]) and not np.any(is_remote[n_remote:])   # remote tiles first
    cnt = [int(np.sum((lay["band_expert"] == el) & (lay["band_dest"] != local))) for el in range(ee - eb)]
    seq = [int(lay["band_expert"][b]) for b in sched[:n_remote]]
    experts = [e for i, e in enumerate(seq) if i == 0 or seq[i - 1] != e]
    assert len(experts) == len(set(experts))                                   # each expert's remote bands together
    assert [cnt[e] for e in experts] == sorted((cnt[e] for e in experts), reverse=True)
    seg = ol.transfer_segments(lay, 2)
    used = np.zeros(nb, dtype=int)
    for fb, n in zip(seg["first_band"], seg["n_bands"]):
        used[fb:fb + n] += 1
    assert np.all(used == 1)
    assert seg["rows"].sum() == lay["recv_rows"].sum()


@pytest.mark.parametrize("T,E,k,eb,ee,S,local,tb", CASES[:4])
def test_segment_copy_reaches_the_receive_definition(T, E, k, eb, ee, S, local, tb):
    # Two constructions of the receive buffer: copying the segments of the
    # padded layout, and the layout-free definition (reading L4).
    idx = _route(T, E, k, 3 * T + E)
    lay = ol.owner_aligned_layout(idx, eb, ee, S, local, tb)
    seg = ol.transfer_segments(lay, 2)
    rng = np.random.default_rng(1)
    o = rng.standard_normal((T * k, 3))
    rs = lay["row_src"]
    O_pad = np.where(rs[:, None] >= 0, o[np.maximum(rs, 0)], 0.0)
    recv = np.full((int(lay["recv_rows"].sum()), 3), np.nan)
    for sr, n, dr in zip(seg["src_row"], seg["rows"], seg["dst_row"]):
        recv[dr:dr + n] = O_pad[sr:sr + n]
    expect = ol.segment_return(idx, eb, ee, S, lambda a: o[a])
    np.testing.assert_array_equal(recv, expect.reshape(recv.shape))
