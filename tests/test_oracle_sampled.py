"""Pin of the oracle's token-restricted path: moe_layer(tokens=...) is what
the full-size GPU parity tests and the CPU baseline compare against, so its
rows must be the rows of the full moe_layer.

Why not bit for bit: the restricted path multiplies fewer rows per expert,
and the BLAS library picks its kernel (and with it the order of the K sum)
from the row count, so a row can move by a few ulps of fp64 (1e-17 absolute
is what a one-row fp8 sample shows). Every mistake this pin is for (a wrong
token mask, a wrong output row q(t), a dropped slot, a slot weight taken
from the wrong assignment) moves a row by O(1) relative, so the bound below,
1e-12 of the row norm, separates the two by ten orders of magnitude. Rows of
tokens with no local expert must be exactly zero, and rows that were not
asked for must be left unset (NaN)."""
import numpy as np
import pytest

import moe_synth
import oracle


CASES = [
    ("bf16_S1", dict()),
    ("bf16_S8", dict(T=64, num_segments=8)),
    ("bf16_share_S8", dict(T=128, E_global=16, e_begin=3, e_end=7, k=4, num_segments=8)),
    ("fp8_S1", dict(dtype="fp8_e4m3", T=256, E_global=16, e_begin=2, e_end=9, k=4)),
    ("fp8_S8", dict(dtype="fp8_e4m3", T=256, E_global=16, e_begin=2, e_end=9, k=4, num_segments=8)),
]


def _samples(cfg, full, rng):
    """Token sets: single tokens, a few, a third of all, and tokens with no local expert."""
    k = cfg.k
    has = np.zeros(cfg.T, bool)
    has[full["row_src"] // k] = True
    with_local = np.flatnonzero(has)
    without = np.flatnonzero(~has)
    sets = [with_local[:1], with_local[-1:], rng.choice(with_local, 5, replace=False),
            np.arange(0, cfg.T, 3)]
    if without.size:
        sets.append(np.concatenate([without[:3], with_local[:2]]))
    return sets, without


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_sampled_rows_equal_full_rows(name, over):
    cfg = moe_synth.make_config("tiny", **over)
    inp = moe_synth.generate(cfg)
    full = oracle.moe_layer(inp, cfg)
    rng = np.random.default_rng(7)
    sets, without = _samples(cfg, full, rng)
    if cfg.e_end - cfg.e_begin < cfg.E_global:
        assert without.size > 0, "the share should leave some tokens without a local expert"
    for toks in sets:
        toks = np.asarray(toks, dtype=np.int64)
        sub = oracle.moe_layer(inp, cfg, tokens=toks)
        q = oracle.y_row_of_token(toks, cfg.T, cfg.num_segments)
        got, want = sub["Y"][q], full["Y"][q]
        assert np.all(np.isfinite(got))
        norms = np.linalg.norm(want, axis=1)
        diff = np.linalg.norm(got - want, axis=1)
        assert np.all(diff <= 1e-12 * norms), (name, toks, (diff / np.maximum(norms, 1e-300)).max())
        # the bookkeeping is computed for every token, whatever the sample
        for key in ("topk_idx", "row_src", "row_dst", "tok_off", "offsets", "comb_w"):
            np.testing.assert_array_equal(sub[key], full[key], err_msg=key)
        # rows outside the sample are not computed
        others = np.setdiff1d(np.arange(cfg.T), q)
        assert np.all(np.isnan(sub["Y"][others]))
    for t in without:
        qz = oracle.y_row_of_token(np.array([t]), cfg.T, cfg.num_segments)
        sub = oracle.moe_layer(inp, cfg, tokens=np.array([t]))
        assert np.all(sub["Y"][qz] == 0.0) and np.all(full["Y"][qz] == 0.0)


def test_sample_mapping_mistake_is_caught():
    """The bound above is not vacuous: taking the output row as t instead of
    q(t) with 8 segments (a plausible mapping slip) breaks it by far."""
    cfg = moe_synth.make_config("tiny", T=64, num_segments=8)
    inp = moe_synth.generate(cfg)
    full = oracle.moe_layer(inp, cfg)
    toks = np.array([3, 10, 41])
    sub = oracle.moe_layer(inp, cfg, tokens=toks)
    q = oracle.y_row_of_token(toks, cfg.T, cfg.num_segments)
    wrong = full["Y"][toks]
    rel = np.linalg.norm(sub["Y"][q] - wrong) / np.linalg.norm(wrong)
    assert rel > 0.1
