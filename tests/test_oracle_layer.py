"""Pins of the oracle's whole-layer computation against the mathematics of
the MoE forward pass (dense special cases, brute force, invariances)."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle


def _tiny(**kw):
    return moe_synth.make_config("tiny", **kw)


def test_single_expert_equals_dense_swiglu_ffn():
    """E=1, k=1 gives weight 1 and the layer reduces to a dense SwiGLU FFN
    (Shazeer, GLU Variants): Y = W2 (silu(W1_gate x) * W1_up x), evaluated
    here independently with torch float64 (no intermediate rounding)."""
    cfg = _tiny(E_global=1, k=1, e_begin=0, e_end=1, d=128, f=192, T=37)
    inp = moe_synth.generate(cfg)
    r = oracle.moe_layer(inp, cfg, h_mode=None)
    x = inp["X"].double()
    W1 = inp["W1"][0].double()
    W2 = inp["W2"][0].double()
    gate = torch.nn.functional.linear(x, W1[:cfg.f])
    up = torch.nn.functional.linear(x, W1[cfg.f:])
    ref = torch.nn.functional.linear(torch.nn.functional.silu(gate) * up, W2).numpy()
    np.testing.assert_allclose(r["Y"], ref, rtol=1e-12, atol=1e-14)
    assert np.all(r["topk_w"] == 1.0)


def test_silu_closed_form_through_layer():
    """One token, d=1 worth of signal: with W1 gate row picking x0 and up row
    picking x1, and W2 picking act, Y = silu(x0) * x1 exactly (x0 = ln 3 gives
    silu = 0.75 ln 3)."""
    cfg = _tiny(E_global=1, k=1, e_begin=0, e_end=1, d=128, f=128, T=1)
    inp = moe_synth.generate(cfg)
    X = torch.zeros(1, 128)
    X[0, 0], X[0, 1] = float(np.log(3.0)), 2.0
    inp["X"] = X.to(torch.bfloat16)
    W1 = torch.zeros(1, 256, 128)
    W1[0, 0, 0] = 1.0          # gate row 0 reads x0
    W1[0, 128, 1] = 1.0        # up row 0 reads x1
    W2 = torch.zeros(1, 128, 128)
    W2[0, 5, 0] = 1.0          # output channel 5 reads act column 0
    inp["W1"], inp["W2"] = W1.to(torch.bfloat16), W2.to(torch.bfloat16)
    r = oracle.moe_layer(inp, cfg, h_mode=None)
    x0 = float(inp["X"][0, 0].float())
    expect = x0 / (1 + np.exp(-x0)) * 2.0
    assert abs(r["Y"][0, 5] - expect) < 1e-15
    assert abs(expect - 0.75 * np.log(3.0) * 2.0) < 2e-2          # bf16-stored ln 3
    assert np.count_nonzero(r["Y"]) == 1


@pytest.mark.parametrize("over", [dict(), dict(e_begin=1, e_end=3), dict(num_segments=4),
                                  dict(k=1), dict(k=4, E_global=4), dict(T=40, num_segments=8, e_begin=2)])
@pytest.mark.parametrize("h_mode", ["bf16", None])
def test_grouped_equals_bruteforce_dense(over, h_mode):
    cfg = _tiny(**over)
    inp = moe_synth.generate(cfg)
    r = oracle.moe_layer(inp, cfg, h_mode=h_mode)
    yb = oracle.moe_layer_bruteforce(inp, cfg, h_mode=h_mode)
    q = oracle.y_row_of_token(np.arange(cfg.T), cfg.T, cfg.num_segments)
    np.testing.assert_allclose(r["Y"][q], yb, rtol=1e-11, atol=1e-15)


def test_fp8_grouped_equals_bruteforce_and_dequant_route():
    """fp8 path: the oracle's own e4m3 decode + block scales agree with torch's
    float8_e4m3fn decode times the expanded scales; grouped == brute force."""
    cfg = _tiny(dtype="fp8_e4m3", T=128, num_segments=8)
    inp = moe_synth.generate(cfg)
    xt = inp["X"].view(torch.float8_e4m3fn).double() * inp["X_scale"].double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    np.testing.assert_array_equal(oracle.decode_x(inp, cfg), xt.numpy())
    w1t = inp["W1"][2].view(torch.float8_e4m3fn).double() * inp["W1_scale"][2].double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    np.testing.assert_array_equal(oracle.decode_expert_weights(inp, cfg, 2)[0], w1t.numpy())
    r = oracle.moe_layer(inp, cfg)
    yb = oracle.moe_layer_bruteforce(inp, cfg)
    q = oracle.y_row_of_token(np.arange(cfg.T), cfg.T, cfg.num_segments)
    np.testing.assert_allclose(r["Y"][q], yb, rtol=1e-11, atol=1e-15)


def test_shares_add_up_to_full_layer():
    """Experts split into disjoint local shares: the partial outputs sum to the
    output with every expert local (the routing is global, reading R3)."""
    cfg = _tiny(E_global=8, k=3, e_end=8, T=48)
    inp = moe_synth.generate(cfg)
    full = oracle.moe_layer(inp, cfg)["Y"]
    acc = np.zeros_like(full)
    for eb, ee in ((0, 3), (3, 4), (4, 8)):
        sub = cfg.replace(e_begin=eb, e_end=ee)
        sinp = dict(inp, W1=inp["W1"][eb:ee], W2=inp["W2"][eb:ee])
        acc += oracle.moe_layer(sinp, sub)["Y"]
    np.testing.assert_allclose(acc, full, rtol=1e-12, atol=1e-16)


def test_token_permutation_invariance():
    cfg = _tiny(T=48, E_global=6, e_end=6, k=2)
    inp = moe_synth.generate(cfg)
    Y = oracle.moe_layer(inp, cfg)["Y"]
    perm = np.random.default_rng(4).permutation(cfg.T)
    pinp = dict(inp, X=inp["X"][perm], logits=inp["logits"][perm])
    Yp = oracle.moe_layer(pinp, cfg)["Y"]
    np.testing.assert_array_equal(Yp, Y[perm])


def test_full_k_is_dense_soft_mixture():
    cfg = _tiny(k=4, E_global=4, T=16)
    inp = moe_synth.generate(cfg)
    Y = oracle.moe_layer(inp, cfg, h_mode=None)["Y"]
    L = inp["logits"].double()
    p = torch.softmax(L, dim=1).numpy()
    X = oracle.decode_x(inp, cfg)
    ref = np.zeros_like(Y)
    for e in range(4):
        W1, W2 = oracle.decode_expert_weights(inp, cfg, e)
        g, u = X @ W1[:cfg.f].T, X @ W1[cfg.f:].T
        ref += p[:, e:e + 1] * ((g * scipy_expit(g) * u) @ W2.T)
    np.testing.assert_allclose(Y, ref, rtol=1e-11, atol=1e-16)


def scipy_expit(z):
    import scipy.special
    return scipy.special.expit(z)


def test_linear_in_w2_and_zero_rows():
    cfg = _tiny(E_global=8, e_begin=0, e_end=2, k=2, T=64)
    inp = moe_synth.generate(cfg)
    r1 = oracle.moe_layer(inp, cfg)
    r2 = oracle.moe_layer(dict(inp, W2=inp["W2"] * 2), cfg)    # power of two: exact in bf16
    np.testing.assert_array_equal(r2["Y"], 2 * r1["Y"])
    none = r1["tok_off"][1:] == r1["tok_off"][:-1]
    assert none.any() and np.all(r1["Y"][none] == 0.0)           # tokens with no local expert


def test_intermediate_rounding_is_applied():
    """The bf16 path rounds H exactly once to bf16: Y(h_mode='bf16') equals
    Linear-2 applied to torch's bf16 cast of the (fp32-representable) act."""
    cfg = _tiny(E_global=1, k=1, e_end=1, T=8)
    inp = moe_synth.generate(cfg)
    X = oracle.decode_x(inp, cfg)
    W1, W2 = oracle.decode_expert_weights(inp, cfg, 0)
    g, u = X @ W1[:cfg.f].T, X @ W1[cfg.f:].T
    act = g * scipy_expit(g) * u
    hr = oracle.round_to_bf16(act)
    assert np.all(np.abs(hr - act) <= np.abs(act) * 2.0 ** -8)
    Y = oracle.moe_layer(inp, cfg)["Y"]
    np.testing.assert_allclose(Y, hr @ W2.T, rtol=1e-13, atol=1e-17)
    assert not np.allclose(Y, act @ W2.T, rtol=1e-6, atol=0)
