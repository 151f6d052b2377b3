"""CPU oracle of the owner-aligned return path (test infrastructure).

TEST INFRASTRUCTURE ONLY: the product path never imports or calls it; it
shares no code with the HIP library.

It follows Cui et al., "Fine-grained Computation-Communication Overlap via
Tile-level Signaling and Scheduling for MoE":
  * Section 3.2.1 (remote-owner-aligned row layout) and the layout half of
    its Algorithm 1: inside every local expert the rows are grouped by the
    rank that owns their token, the remote ranks in ascending order and this
    rank's own group last; each remote group is padded with zero rows up to a
    multiple of the tile height tb_M, so every row band of tb_M rows has one
    owner. The own (local) group is not padded.
  * Section 3.2.2 and the schedule half of Algorithm 1 (remote-first tile
    schedule): experts sorted by their number of remote row bands, most
    first; every remote band of those experts in that order, then the local
    bands expert by expert.
  * Section 3.2.3 (combine plan): per band, the destination rank, the row
    offset inside that rank's receive buffer and the number of valid rows.
  * Section 3.3.2 and Figure 3b (segment-granular transfer): within one
    destination group, the first and the last segment hold one band each and
    the middle segments up to x bands.
  * Section 4.5: at most (W-1)(tb_M-1) padded rows for W ranks.

Readings where the page leaves a step open:
  L1  the owner of token t is rank t mod S (the token -> segment map of the
      eight-segment workloads), S = the number of ranks (destinations);
  L2  rows inside a group keep ascending assignment id a = t*k + j, as in the
      unpadded dispatch;
  L3  ties in the expert sort keep ascending local expert index;
  L4  the receive buffer of rank s holds this rank's rows for s in (expert,
      assignment id) order; one buffer holds the S regions one after another;
  L5  the local group is a transfer too (on one GPU every destination is
      local HBM), copied band by band with the same segment rule, so the
      receive buffer is complete; the plan still marks its bands local-only;
  L6  the Section 4.5 bound is read per expert (each expert has at most W-1
      padded group boundaries); a rank with E_l experts pads at most
      E_l (W-1)(tb_M-1) rows.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

__all__ = ["owner_aligned_layout", "remote_first_schedule", "transfer_segments", "segment_return",
           "owner_of_token"]


def owner_of_token(t, S: int):
    """Reading L1: rank t mod S owns token t."""
    return np.asarray(t) % S


def owner_aligned_layout(idx, e_begin: int, e_end: int, S: int, local: int, tb_M: int) -> Dict[str, np.ndarray]:
    """Row layout of Section 3.2.1 / Algorithm 1 (layout part).

    Returns row_src (assignment id of every padded row, -1 for a zero row),
    expert_off [E_l + 1], group_rows / group_off [E_l, S] (valid rows and
    first padded row of the group of expert e for rank s) and the band table
    (expert, dest, first row, valid rows, receive offset), in layout order.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    El = e_end - e_begin
    assert 0 <= local < S and tb_M >= 1
    flat = idx.reshape(-1)
    owner = owner_of_token(np.arange(T * k) // k, S)
    order = [r for r in range(S) if r != local] + [local]      # remote ranks ascending, own rank last
    row_src = []
    expert_off = [0]
    group_rows = np.zeros((El, S), dtype=np.int64)
    group_off = np.zeros((El, S), dtype=np.int64)
    recv_rows = np.zeros(S, dtype=np.int64)                       # rows already placed per destination
    bands = []
    for el in range(El):
        e = e_begin + el
        for r in order:
            g = np.nonzero((flat == e) & (owner == r))[0]         # ascending assignment id (L2)
            n = len(g)
            padded = n if r == local else -(-n // tb_M) * tb_M    # remote groups to a tb_M multiple
            first = len(row_src)
            group_rows[el, r] = n
            group_off[el, r] = first
            row_src.extend(int(a) for a in g)
            row_src.extend([-1] * (padded - n))
            for b0 in range(0, padded, tb_M):
                valid = max(0, min(tb_M, n - b0))
                bands.append((el, r, first + b0, valid, int(recv_rows[r]) + b0))
            recv_rows[r] += n
        expert_off.append(len(row_src))
    bt = np.array(bands, dtype=np.int64).reshape(-1, 5)
    return {
        "row_src": np.array(row_src, dtype=np.int64),
        "expert_off": np.array(expert_off, dtype=np.int64),
        "group_rows": group_rows,
        "group_off": group_off,
        "band_expert": bt[:, 0], "band_dest": bt[:, 1], "band_row": bt[:, 2],
        "band_valid": bt[:, 3], "band_recv_off": bt[:, 4],
        "recv_rows": recv_rows,
        "recv_start": np.concatenate([[0], np.cumsum(recv_rows)[:-1]]).astype(np.int64),
        "R": len(row_src), "local": local, "S": S, "tb_M": tb_M,
    }


def remote_first_schedule(lay) -> np.ndarray:
    """Band order of Section 3.2.2 / Algorithm 1 (schedule part): experts by
    descending remote band count (ties: ascending expert, L3), all their remote
    bands first; then every local band in expert order."""
    be, bd = lay["band_expert"], lay["band_dest"]
    local = lay["local"]
    El = len(lay["expert_off"]) - 1
    remote_cnt = [int(np.sum((be == el) & (bd != local))) for el in range(El)]
    experts = sorted(range(El), key=lambda el: (-remote_cnt[el], el))
    sched = []
    for el in experts:
        sched.extend(int(b) for b in np.nonzero((be == el) & (bd != local))[0])
    for el in range(El):
        sched.extend(int(b) for b in np.nonzero((be == el) & (bd == local))[0])
    return np.array(sched, dtype=np.int64)


def transfer_segments(lay, x: int) -> Dict[str, np.ndarray]:
    """Segments of Section 3.3.2 / Figure 3b: in each (expert, destination)
    group of n bands, the first and the last segment are one band each and the
    middle ones take up to x bands. A segment copies its valid rows
    (contiguous in the layout and in the receive buffer). Segments are listed
    in the order their first band appears in the remote-first schedule."""
    assert x >= 1
    sched = remote_first_schedule(lay)
    pos = np.empty(len(sched), dtype=np.int64)
    pos[sched] = np.arange(len(sched))
    be, bd = lay["band_expert"], lay["band_dest"]
    segs = []
    seen = set()
    for b in sched:
        key = (int(be[b]), int(bd[b]))
        if key in seen:
            continue
        seen.add(key)
        members = [int(i) for i in np.nonzero((be == key[0]) & (bd == key[1]))[0]]
        n = len(members)
        if n <= 2:
            parts = [[m] for m in members]
        else:
            mid = members[1:-1]
            parts = [[members[0]]] + [mid[i:i + x] for i in range(0, len(mid), x)] + [[members[-1]]]
        for part in parts:
            valid = int(sum(lay["band_valid"][i] for i in part))
            segs.append((part[0], len(part), key[1], int(lay["band_row"][part[0]]), valid,
                         int(lay["recv_start"][key[1]] + lay["band_recv_off"][part[0]]),
                         int(key[1] != lay["local"])))
    st = np.array(segs, dtype=np.int64).reshape(-1, 7)
    return {"first_band": st[:, 0], "n_bands": st[:, 1], "dest": st[:, 2], "src_row": st[:, 3],
            "rows": st[:, 4], "dst_row": st[:, 5], "remote": st[:, 6]}


def segment_return(idx, e_begin: int, e_end: int, S: int, o_of_assignment) -> np.ndarray:
    """What the receive buffer holds once every transfer is done (reading L4),
    defined without the layout: region s lists, for every local expert in
    ascending order, o[a] of its assignments owned by rank s in ascending a.
    o_of_assignment maps an assignment id to its expert-output row."""
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1)
    rows = []
    for s in range(S):
        for e in range(e_begin, e_end):
            for a in range(T * k):
                if flat[a] == e and (a // k) % S == s:
                    rows.append(o_of_assignment(a))
    if not rows:
        return np.zeros((0, 0))
    return np.stack(rows)
