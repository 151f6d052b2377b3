"""CPU oracle for one GPU's share of a Mixture-of-Experts layer (test infrastructure).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or calls
this module: only the tests, the package-level smoke check and the CPU
baseline leg of the benchmark may use it. It shares no code with the HIP
library (no kernels, headers, helpers or tables); the only module both sides
see is the seeded input generator `moe_synth`, which holds no layer
arithmetic.

What it computes, step by step, follows the forward pass as the pages define
it:

  * "Fine-grained Computation-Communication Overlap via Tile-level Signaling
    and Scheduling for MoE" (Cui et al.), Section 2.1: (1) routing produces
    per-token expert assignments and gate weights from a probability
    distribution over experts, top-k kept; (2) dispatch sends each token to
    its experts; (3) each expert runs on its tokens; (4)/(5) outputs return to
    the token's owner, which forms the gate-weighted sum.
  * "X-Stage: An Overlooked Pipeline Stage for Communication-Computation
    Overlap in DiT Inference" (Xian et al.), Section 2.2 (MegaMoE Execution):
    each expert is a two-layer FFN, Linear-1 (hidden -> intermediate), an
    activation such as SwiGLU, Linear-2 (intermediate -> hidden); Combine
    aggregates the top-k results with the router weights.

Readings where the pages leave a step open (each is also stated where used):
  R1  top-k order: descending logit, ties to the lower expert index
      (-0.0 ties +0.0); weights are the softmax over the k selected logits.
  R2  W1[e] is [2f, d] (out, in); rows [0, f) are the gate, rows [f, 2f) the
      up projection; act = silu(gate) * up; W2[e] is [d, f] (out, in).
  R3  the local share is experts [e_begin, e_end): routing is over all
      E_global logits, only local assignments are computed, Y is this share's
      partial sum, rows with no local assignment are zero.
  R4  expert-contiguous row order (dispatch permutation) is ascending
      assignment id a = t*k + j within each expert (a stable counting sort).
  R5  token order of the combine buffer: with S destination segments token t
      lands on Y-row q(t) = (t mod S) * (T/S) + t div S; rows ordered by
      (q(t), j).
  R6  the intermediate H is rounded to the Linear-2 operand type before
      Linear-2: bf16 (round to nearest even), or e4m3 with one fp32 scale per
      row and 128 consecutive columns (scale = amax/448, 1 if amax = 0).
  R7  gate weights are applied in the combine step, not inside Linear-2.

Precision: fp64 throughout except the roundings R6 forces and the fp32
storage of block scales. Inputs are the exact bf16 / e4m3 / MXFP4 bit
patterns the GPU receives. fp64 is a reading too: the target names an fp32
oracle; fp64 is the same definition with less rounding of its own, so its
distance to the GPU result is the GPU's error alone.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "round_to_bf16",
    "e4m3_bits_to_f64", "f64_to_e4m3_bits", "round_to_e4m3",
    "quantize_rows_e4m3", "e2m1_to_f64", "e8m0_to_f64", "decode_mxfp4",
    "route_topk", "dispatch", "swiglu_expert",
    "round_intermediate", "combine", "decode_x", "decode_expert_weights",
    "moe_layer", "moe_layer_bruteforce", "y_row_of_token",
]


# ----------------------------------------------------------------------------
# Number formats, written from their definitions.
#   bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits; the upper half
#             of an IEEE binary32.
#   OCP FP8 E4M3 ("E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
#             exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN;
#             no infinities; largest finite 448 = 1.75 * 2^8.
# ----------------------------------------------------------------------------

def _round_to_format(x, mant_bits: int, emin: int) -> np.ndarray:
    """Round fp64 values to a binary format with `mant_bits` stored mantissa
    bits and minimum normal exponent `emin`, to nearest, ties to even, with
    unbounded exponent range above (overflow handled by the caller).

    Every value with |x| in [2^e, 2^(e+1)) (e >= emin) sits on a grid of
    quantum 2^(e - mant_bits); below 2^emin the grid is that of emin
    (subnormals). Scaling by a power of two is exact, so rint (which rounds
    half to even) performs the rounding exactly."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)              # ax = m * 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, emin)      # floor(log2 ax), clamped to the subnormal grid
    quantum = np.ldexp(1.0, e - mant_bits)
    with np.errstate(invalid="ignore"):
        r = np.rint(ax / quantum) * quantum
    return np.copysign(r, x)


def round_to_bf16(x) -> np.ndarray:
    """Nearest bf16 value (ties to even) of fp64 input, as fp64; overflow -> inf."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_format(x, 7, -126)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, x), r)
    return np.where(np.isnan(x), np.nan, r)


def f64_to_bf16_bits(x) -> np.ndarray:
    r = round_to_bf16(x)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(r), np.uint16(0x7FC0), bits).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


E4M3_MAX = 448.0


def round_to_e4m3(x) -> np.ndarray:
    """Nearest E4M3FN value (ties to even), saturating to +-448, as fp64."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_format(x, 3, -6)
    r = np.clip(r, -E4M3_MAX, E4M3_MAX)
    return np.where(np.isnan(x), np.nan, r)


def f64_to_e4m3_bits(x) -> np.ndarray:
    r = round_to_e4m3(x)
    sign = np.signbit(r).astype(np.uint8) << 7
    ar = np.abs(r)
    out = np.zeros(r.shape, dtype=np.uint8)
    sub = ar < 2.0 ** -6
    out = np.where(sub, np.rint(ar / 2.0 ** -9).astype(np.int64), out)
    with np.errstate(divide="ignore"):
        _, e = np.frexp(np.where(sub, 1.0, ar))
    E = e - 1 + 7                                  # biased exponent field
    mant = np.rint((np.where(sub, 1.0, ar) / np.ldexp(1.0, E - 7) - 1.0) * 8.0).astype(np.int64)
    normal = (E << 3) | mant
    out = np.where(sub, out, normal).astype(np.uint8) | sign
    return np.where(np.isnan(r), np.uint8(0x7F), out).astype(np.uint8)


def e4m3_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    E = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(E == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, E - 7))
    val = np.where((E == 15) & (m == 7), np.nan, val)
    return s * val


def quantize_rows_e4m3(a: np.ndarray, block: int = 128):
    """Reading R6 for the fp8 path: per row, per `block` consecutive columns,
    scale = amax / 448 stored in fp32 (1 when the block is all zero), code =
    nearest e4m3 of a / scale. Returns (codes uint8, scales fp32 [rows, cols/block],
    dequantised fp64)."""
    a = np.asarray(a, dtype=np.float64)
    n, c = a.shape
    assert c % block == 0
    ab = a.reshape(n, c // block, block)
    amax = np.abs(ab).max(axis=2).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    codes = f64_to_e4m3_bits(ab / scale[:, :, None].astype(np.float64))
    deq = e4m3_bits_to_f64(codes) * scale[:, :, None].astype(np.float64)
    return codes.reshape(n, c), scale, deq.reshape(n, c)


# ----------------------------------------------------------------------------
# MXFP4 weights (the low-bit weight format of the W4A8 workload), written
# from the OCP Microscaling (MX) formats definition:
#   E2M1 element: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent
#             field 0 is subnormal (m * 0.5); no infinities or NaN; the
#             magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
#   E8M0 scale: 8 exponent bits, bias 127, no sign or mantissa: 2^(e - 127);
#             the code 0xFF is NaN.
#   A block is 32 consecutive elements along K sharing one E8M0 scale:
#             value = scale * element.
# Storage (this library's reading, stated in the workload): a weight row of
# K elements is K/2 bytes, byte j holding element 2j in its low nibble and
# 2j + 1 in its high nibble; the scales are one byte per row and 32-element
# block, [rows, K/32].
# ----------------------------------------------------------------------------

def e2m1_to_f64(codes) -> np.ndarray:
    """Value of 4-bit E2M1 codes (0..15)."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    E = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(E == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, E - 1))
    return s * mag


def e8m0_to_f64(codes) -> np.ndarray:
    """Value of E8M0 scale bytes: 2^(e - 127), NaN for 0xFF."""
    e = np.asarray(codes).astype(np.int64)
    return np.where(e == 0xFF, np.nan, np.ldexp(1.0, e - 127))


def decode_mxfp4(packed, scales, block: int = 32) -> np.ndarray:
    """Packed MXFP4 rows [rows, K/2] uint8 with E8M0 scales [rows, K/block]
    -> fp64 [rows, K]."""
    b = np.asarray(packed).astype(np.uint8)
    lo, hi = b & 0xF, b >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(b.shape[0], b.shape[1] * 2)
    sc = np.repeat(e8m0_to_f64(scales), block, axis=-1)
    return e2m1_to_f64(codes) * sc


# ----------------------------------------------------------------------------
# (1) Routing: Cui et al. Section 2.1 step (1); configs: softmax over the
# top-k, renormalised. Reading R1.
# ----------------------------------------------------------------------------

def route_topk(logits, k: int):
    """Top-k experts per token and their gate weights.

    logits: [T, E] fp32. Returns idx [T, k] int32 (slot order: descending
    logit, ties to the lower index), w [T, k] fp64 = exp(l_j - l_max) /
    sum_i exp(l_i - l_max) over the k selected logits, and the global
    per-expert assignment counts [E] (they sum to T*k)."""
    L = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = L.shape
    assert 1 <= k <= E
    expert_ids = np.broadcast_to(np.arange(E), L.shape)
    # lexsort: last key is primary. -0.0 and +0.0 compare equal, so they tie.
    order = np.lexsort((expert_ids, -L), axis=-1)
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    counts_global = np.bincount(idx.reshape(-1), minlength=E).astype(np.int64)
    return idx, w, counts_global


# ----------------------------------------------------------------------------
# (2) Dispatch on one GPU: Cui et al. Section 2.1 step (2) becomes a
# permutation of rows into expert-contiguous order. Readings R3, R4, R5.
# ----------------------------------------------------------------------------

def y_row_of_token(t, T: int, S: int):
    """Reading R5: token t's output row when the output is S segments of T/S rows."""
    t = np.asarray(t)
    return (t % S) * (T // S) + t // S


def dispatch(idx, w, e_begin: int, e_end: int, num_segments: int = 1) -> Dict[str, np.ndarray]:
    """Row bookkeeping for the local share.

    counts[e]  local assignments of local expert e (e relative to e_begin)
    offsets    exclusive prefix sum of counts, offsets[E_l] = A
    row_src[r] assignment id a = t*k + j of expert-ordered row r; rows of
               one expert in ascending a
    tok_off[q] first token-order slot of output row q (length T + 1)
    row_dst[r] token-order slot of expert-ordered row r
    comb_w[p]  gate weight of the assignment at token-order slot p
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    S = num_segments
    assert T % S == 0
    El = e_end - e_begin
    a_all = np.arange(T * k, dtype=np.int64)
    e_all = idx.reshape(-1).astype(np.int64)
    local = (e_all >= e_begin) & (e_all < e_end)
    a_loc = a_all[local]
    e_loc = e_all[local] - e_begin
    A = int(a_loc.size)

    counts = np.bincount(e_loc, minlength=El).astype(np.int64)
    offsets = np.zeros(El + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_src = a_loc[np.argsort(e_loc, kind="stable")]

    t_loc, j_loc = a_loc // k, a_loc % k
    q_loc = y_row_of_token(t_loc, T, S)
    tok_list = a_loc[np.lexsort((j_loc, q_loc))]        # assignment ids in token order
    slot_of = np.full(T * k, -1, dtype=np.int64)
    slot_of[tok_list] = np.arange(A)
    row_dst = slot_of[row_src]
    tok_off = np.zeros(T + 1, dtype=np.int64)
    tok_off[1:] = np.cumsum(np.bincount(q_loc, minlength=T))
    comb_w = np.asarray(w, dtype=np.float64).reshape(-1)[tok_list]
    return dict(counts=counts, offsets=offsets, row_src=row_src, row_dst=row_dst,
                tok_off=tok_off, comb_w=comb_w, A=A, tok_list=tok_list)


# ----------------------------------------------------------------------------
# (3) Expert computation: X-Stage Section 2.2 (Linear-1, SwiGLU, Linear-2);
# SwiGLU per Shazeer, "GLU Variants Improve Transformer". Readings R2, R6.
# ----------------------------------------------------------------------------

def round_intermediate(a: np.ndarray, mode: Optional[str], block: int = 128) -> np.ndarray:
    """Reading R6: 'bf16', 'e4m3' (per row, per `block` columns) or None (no rounding)."""
    if mode is None:
        return a
    if mode == "bf16":
        return round_to_bf16(a)
    if mode == "e4m3":
        return quantize_rows_e4m3(a, block)[2]
    raise ValueError(mode)


def swiglu_expert(x: np.ndarray, W1e: np.ndarray, W2e: np.ndarray, h_mode: Optional[str],
                  block: int = 128) -> np.ndarray:
    """o = W2e @ round(silu(W1e[:f] @ x) * (W1e[f:] @ x)) for each row x of `x`."""
    f = W1e.shape[0] // 2
    h = x @ W1e.T
    gate, up = h[:, :f], h[:, f:]
    with np.errstate(over="ignore"):
        act = gate / (1.0 + np.exp(-gate)) * up
    return round_intermediate(act, h_mode, block) @ W2e.T


# ----------------------------------------------------------------------------
# (4)+(5) Combine: Cui et al. Section 2.1 step (5), gate-weighted sum of the
# returned expert outputs; X-Stage Section 2.2. Reading R7.
# ----------------------------------------------------------------------------

def combine(buf: np.ndarray, tok_off: np.ndarray, comb_w: np.ndarray, rows=None) -> np.ndarray:
    """Y[q] = sum over slots p in [tok_off[q], tok_off[q+1]) of comb_w[p] * buf[p],
    in slot order; rows with no slot are zero. `rows` limits the output rows
    computed (others NaN)."""
    T = tok_off.size - 1
    d = buf.shape[1]
    Y = np.zeros((T, d)) if rows is None else np.full((T, d), np.nan)
    for q in (range(T) if rows is None else rows):
        acc = np.zeros(d)
        for p in range(tok_off[q], tok_off[q + 1]):
            acc = acc + comb_w[p] * buf[p]
        Y[q] = acc
    return Y


# ----------------------------------------------------------------------------
# Input decoding (storage formats of moe_synth) and the whole layer.
# ----------------------------------------------------------------------------

def _np(t) -> np.ndarray:
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if str(t.dtype) == "torch.bfloat16":
            import torch
            t = t.view(torch.int16)
        return t.numpy()
    return np.asarray(t)


def _block_expand(scale: np.ndarray, block: int) -> np.ndarray:
    return np.repeat(np.repeat(scale.astype(np.float64), block, axis=-2), block, axis=-1)


def decode_x(inp, cfg, tokens=None) -> np.ndarray:
    """X as fp64 [T, d] (or only the rows in `tokens`)."""
    X = _np(inp["X"])
    if cfg.dtype in ("fp8_e4m3", "w4a8_mxfp4"):
        v = e4m3_bits_to_f64(X) * _block_expand(_np(inp["X_scale"]), cfg.quant_block)
    else:
        v = bf16_bits_to_f64(X.view(np.uint16))
    return v if tokens is None else v[np.asarray(tokens)]


def decode_expert_weights(inp, cfg, e_local: int):
    """(W1[e] [2f, d], W2[e] [d, f]) as fp64 for local expert e_local."""
    out = []
    for name in ("W1", "W2"):
        W = inp[name][e_local]
        Wn = _np(W)
        if cfg.dtype == "w4a8_mxfp4":
            out.append(decode_mxfp4(Wn, _np(inp[name + "_scale"][e_local])))
        elif cfg.dtype == "fp8_e4m3":
            out.append(e4m3_bits_to_f64(Wn) * _block_expand(_np(inp[name + "_scale"][e_local]), cfg.quant_block))
        else:
            out.append(bf16_bits_to_f64(Wn.view(np.uint16)))
    return tuple(out)


def default_h_mode(cfg) -> str:
    return "e4m3" if cfg.dtype in ("fp8_e4m3", "w4a8_mxfp4") else "bf16"


def moe_layer(inp, cfg, h_mode="auto", tokens: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """The whole local share: route -> dispatch -> per-expert SwiGLU FFN ->
    combine. With `tokens`, only those tokens' output rows are computed (the
    bookkeeping arrays are always complete). Returns every intermediate and
    Y [T, d] fp64 (rows in output-row order q)."""
    if h_mode == "auto":
        h_mode = default_h_mode(cfg)
    logits = _np(inp["logits"])
    idx, w, counts_global = route_topk(logits, cfg.k)
    disp = dispatch(idx, w, cfg.e_begin, cfg.e_end, cfg.num_segments)
    T, k, d = cfg.T, cfg.k, cfg.d
    want = np.ones(T, dtype=bool)
    if tokens is not None:
        want[:] = False
        want[np.asarray(tokens)] = True
    buf = np.zeros((disp["A"], d))
    offsets, row_src, row_dst = disp["offsets"], disp["row_src"], disp["row_dst"]
    X_all = None
    for e in range(cfg.E_local):
        rows = np.arange(offsets[e], offsets[e + 1])
        toks = row_src[rows] // k
        rows, toks = rows[want[toks]], toks[want[toks]]
        if rows.size == 0:
            continue
        if X_all is None:
            X_all = decode_x(inp, cfg)
        W1e, W2e = decode_expert_weights(inp, cfg, e)
        buf[row_dst[rows]] = swiglu_expert(X_all[toks], W1e, W2e, h_mode, cfg.quant_block)
    out_rows = None if tokens is None else y_row_of_token(np.asarray(tokens), T, cfg.num_segments)
    Y = combine(buf, disp["tok_off"], disp["comb_w"], rows=out_rows)
    return dict(topk_idx=idx, topk_w=w, counts_global=counts_global, Y=Y, combine_buf=buf, **disp)


def moe_layer_bruteforce(inp, cfg, h_mode="auto") -> np.ndarray:
    """Dense per-token evaluation in fp64 that uses neither the dispatch
    permutation nor the combine bookkeeping: every local expert's FFN is
    evaluated on every token and multiplied by a gate that is zero unless
    the expert is among the token's top-k. Expert e is in the top-k iff fewer
    than k experts e' beat it, where e' beats e when l[e'] > l[e] or
    (l[e'] == l[e] and e' < e). Returns Y [T, d] in token order t (not q)."""
    if h_mode == "auto":
        h_mode = default_h_mode(cfg)
    L = _np(inp["logits"]).astype(np.float32).astype(np.float64)
    X = decode_x(inp, cfg)
    T, E = L.shape
    Y = np.zeros((T, cfg.d))
    ids = np.arange(E)
    gate = np.zeros((T, E))
    for t in range(T):
        l = L[t]
        beaten_by = np.array([np.sum((l > l[e]) | ((l == l[e]) & (ids < e))) for e in range(E)])
        sel = beaten_by < cfg.k
        m = l[sel].max()
        z = np.where(sel, np.exp(l - m), 0.0)
        gate[t] = z / z.sum()
    for e in range(cfg.e_begin, cfg.e_end):
        W1e, W2e = decode_expert_weights(inp, cfg, e - cfg.e_begin)
        Y += gate[:, e:e + 1] * swiglu_expert(X, W1e, W2e, h_mode, cfg.quant_block)
    return Y
