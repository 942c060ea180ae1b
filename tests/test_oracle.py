"""Pins for the float64 oracle: each checks it against something other than itself.

Pins used: hand-worked fixtures (tests/golden), the explicit O(N^2) weight definition, closed forms
of special cases (t = 1, t = 2, constant logits, aligned q/k with identical v), gate limits that
reduce to a library softmax, the zero-sum property, invariances (causality, linearity, scale,
relative-position RoPE), the Taylor meaning of delta, and decode continuity.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import zeros_ref as R
from synth import CONFIGS, make_inputs

TOL = 1e-12


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


def small_inputs(B=2, H=3, N=24, d=8, du=8, seed=11, tau_uniform=True, u_scale=1.0):
    wl = CONFIGS[1].with_(B=B, H=H, N=N, d=d, d_u=du, seed=seed, tau_uniform=tau_uniform)
    return make_inputs(wl, u_scale=u_scale)


# ---------------------------------------------------------------- hand-worked fixtures

def test_logits_hand_fixture(golden_dir):
    with open(os.path.join(golden_dir, "logits_hand.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        u = np.array(case["u"])[:, None]
        tau = np.log(case["exp_tau"])
        s = R.deviation_logits_causal(u, np.array(case["mu"]), np.array(tau))
        np.testing.assert_allclose(s, case["s"], rtol=1e-14, atol=1e-14)


def test_t2_hand_fixture(golden_dir):
    with open(os.path.join(golden_dir, "t2_hand.json")) as f:
        fx = json.load(f)
    x = {key: np.array(val)[None, None] for key, val in fx["inputs"].items()}
    for key in ("q", "k", "v", "u"):
        x[key] = x[key][..., None]
    args = dict(q=x["q"], k=x["k"], v=x["v"], u=x["u"], mu=np.zeros((1, 1)), tau=np.zeros(1),
                g1=x["g1"], gh=x["gh"])
    for fn in (R.causal_forward, R.causal_brute_force):
        o = fn(**args)[0, 0, :, 0]
        np.testing.assert_allclose(o, fx["o"], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- recurrence vs definition

@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 64, 16, 16), (2, 3, 37, 8, 8), (1, 2, 50, 32, 32),
                                   (1, 1, 20, 16, 8)])
def test_recurrence_matches_explicit_weights(shape, rope):
    B, H, N, d, du = shape
    x = small_inputs(B, H, N, d, du, seed=100 + N)
    o = R.causal_forward(**x, rope=rope)
    ob = R.causal_brute_force(**x, rope=rope)
    assert rel(o, ob) < TOL


def test_config1_matches_explicit_weights():
    x = make_inputs(CONFIGS[1])
    assert rel(R.causal_forward(**x), R.causal_brute_force(**x)) < TOL


@pytest.mark.parametrize("rope", [False, True])
def test_encoder_closed_form_matches_explicit_weights(rope):
    x = small_inputs(3, 2, 41, 16, 16, seed=5)
    assert rel(R.encoder_forward(**x, rope=rope), R.encoder_brute_force(**x, rope=rope)) < TOL


# ---------------------------------------------------------------- zero-sum and special cases

def test_explicit_weights_sum_to_zero():
    x = small_inputs(2, 2, 30, 8, 8, seed=3)
    s = R.deviation_logits_causal(x["u"], x["mu"], x["tau"])
    W = R.explicit_weights_causal(s, x["g1"], x["gh"])
    assert np.max(np.abs(W.sum(-1))) < TOL
    assert np.all(np.triu(np.ones((30, 30)), 1)[None, None] * W == 0)       # causal mask
    We = R.explicit_weights_encoder(s, x["g1"], x["gh"])
    assert np.max(np.abs(We.sum(-1))) < TOL


def test_coefficients_zero_sum_form():
    rng = np.random.default_rng(0)
    t = rng.integers(1, 5000, size=200).astype(float)
    E = rng.uniform(1.0, 3.0, size=200) * t
    P = rng.normal(size=200) * t
    s1, sh = rng.uniform(size=200), rng.uniform(size=200)
    a, b, g = R.coefficients(t, E, P, s1, sh)
    resid = a * E + b * P + g * t
    assert np.max(np.abs(resid)) < 1e-12


def test_first_output_is_zero():
    x = small_inputs(2, 2, 5, 8, 8, seed=9)
    o = R.causal_forward(**x)
    assert np.max(np.abs(o[..., 0, :])) < 1e-12 * np.max(np.abs(x["v"]))


def test_identical_values_aligned_directions_give_zero():
    N, d = 40, 8
    rng = np.random.default_rng(1)
    c = rng.normal(size=d)
    vvec = rng.normal(size=d)
    q = np.tile(c, (1, 1, N, 1)) * rng.uniform(0.5, 2.0, size=(1, 1, N, 1))
    k = np.tile(c, (1, 1, N, 1)) * rng.uniform(0.5, 2.0, size=(1, 1, N, 1))
    v = np.tile(vvec, (1, 1, N, 1))
    u = rng.normal(size=(1, 1, N, d))
    g = rng.normal(size=(1, 1, N))
    o = R.causal_forward(q, k, v, u, rng.normal(size=(1, d)) * 0.1, np.zeros(1), g, -g)
    assert np.max(np.abs(o)) < TOL


def test_constant_logits_give_zero():
    x = small_inputs(1, 2, 30, 8, 8, seed=4)
    x["u"] = np.zeros_like(x["u"])
    assert np.max(np.abs(R.causal_forward(**x))) == 0.0
    assert np.max(np.abs(R.encoder_forward(**x))) == 0.0


# ---------------------------------------------------------------- gate limits

def _cos(x, rope=False):
    qh, kh = R.angular_vectors(x["q"], x["k"], rope)
    return qh @ np.swapaxes(kh, -1, -2)


def test_gates_closed_reduce_to_zero():
    x = small_inputs(1, 2, 25, 8, 8, seed=12)
    x["g1"] = np.full_like(x["g1"], -1000.0)
    x["gh"] = np.full_like(x["gh"], -1000.0)
    assert np.max(np.abs(R.causal_forward(**x))) < 1e-300


def test_gates_open_reduce_to_softmax_minus_uniform():
    """sigma1 = sigmah = 1: w = softmax - 1/t, built here with scipy's softmax."""
    x = small_inputs(1, 2, 25, 8, 8, seed=13)
    x["g1"] = np.full_like(x["g1"], 1000.0)
    x["gh"] = np.full_like(x["gh"], 1000.0)
    o = R.causal_forward(**x)
    s = R.deviation_logits_causal(x["u"], x["mu"], x["tau"])
    cos = _cos(x)
    N = s.shape[-1]
    ref = np.zeros_like(o)
    for h in range(2):
        for ti in range(N):
            w = sp_softmax(s[0, h, :ti + 1]) - 1.0 / (ti + 1)
            ref[0, h, ti] = (w * cos[0, h, ti, :ti + 1]) @ x["v"][0, h, :ti + 1].astype(float)
    assert rel(o, ref) < TOL


def test_first_order_only_gate():
    """sigma1 = 1, sigmah = 0: w = (s_i - mean_{j<=t} s_j)/t."""
    x = small_inputs(1, 1, 25, 8, 8, seed=14)
    x["g1"] = np.full_like(x["g1"], 1000.0)
    x["gh"] = np.full_like(x["gh"], -1000.0)
    o = R.causal_forward(**x)
    s = R.deviation_logits_causal(x["u"], x["mu"], x["tau"])[0, 0]
    cos = _cos(x)[0, 0]
    ref = np.zeros_like(o[0, 0])
    for ti in range(s.size):
        w = (s[:ti + 1] - s[:ti + 1].mean()) / (ti + 1)
        ref[ti] = (w * cos[ti, :ti + 1]) @ x["v"][0, 0, :ti + 1].astype(float)
    assert rel(o[0, 0], ref) < TOL


def test_delta_is_first_order_taylor_term():
    """softmax(eps*s) = 1/t + eps*delta/t + O(eps^2): the residual term scales as eps^2."""
    rng = np.random.default_rng(2)
    s = rng.normal(size=12)
    g_open = np.full((12,), 1000.0)
    res = []
    for eps in (1e-2, 1e-3):
        W = R.explicit_weights_causal(eps * s, -g_open, g_open)   # sigma1 = 0, sigmah = 1: w = eps_res
        res.append(np.max(np.abs(W)))
    assert res[0] / res[1] == pytest.approx(100.0, rel=0.05)


# ---------------------------------------------------------------- logits

def test_logit_first_step_closed_form():
    x = small_inputs(2, 3, 10, 8, 8, seed=21)
    s = R.deviation_logits_causal(x["u"], x["mu"], x["tau"])
    u1 = x["u"][..., 0, :].astype(float)
    et = np.exp(x["tau"].astype(float))[None, :, None]
    ubar1 = (et * x["mu"][None] + u1) / (et + 1.0)
    ref = -np.sum(u1 * ubar1, -1) / np.sqrt(8.0)
    np.testing.assert_allclose(s[..., 0], ref, rtol=1e-14)


def test_logit_tau_limits():
    rng = np.random.default_rng(5)
    u = rng.normal(size=(1, 30, 4))
    mu = rng.normal(size=(1, 4))
    # tau -> -inf: ubar_i becomes the plain running mean of u_1..u_i
    s_lo = R.deviation_logits_causal(u, mu, np.array([-60.0]))
    run_mean = np.array([u[0, :i + 1].mean(0) for i in range(30)])
    np.testing.assert_allclose(s_lo[0], -np.sum(u[0] * run_mean, -1) / 2.0, rtol=1e-12, atol=1e-14)
    # tau -> +inf: ubar_i -> mu
    s_hi = R.deviation_logits_causal(u, mu, np.array([60.0]))
    np.testing.assert_allclose(s_hi[0], -(u[0] @ mu[0]) / 2.0, rtol=1e-12, atol=1e-14)


def test_encoder_logits_equal_last_causal_logit_mean():
    """Encoder ubar equals the causal ubar_N: the last causal logit matches."""
    x = small_inputs(1, 2, 17, 8, 8, seed=22)
    sc = R.deviation_logits_causal(x["u"], x["mu"], x["tau"])
    se = R.deviation_logits_encoder(x["u"], x["mu"], x["tau"])
    np.testing.assert_allclose(se[..., -1], sc[..., -1], rtol=1e-13)


# ---------------------------------------------------------------- RoPE

def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(5, 16))
    pos = np.array([0.0, 1.0, 7.0, 100.0, 16383.0])
    out = R.rope_rotate(x, pos, 10000.0)
    z = x[:, 0::2] + 1j * x[:, 1::2]
    theta = 10000.0 ** (-np.arange(8) * 2.0 / 16)
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    np.testing.assert_allclose(out[:, 0::2], zr.real, atol=1e-12)
    np.testing.assert_allclose(out[:, 1::2], zr.imag, atol=1e-12)
    np.testing.assert_array_equal(R.rope_rotate(x, np.zeros(5), 10000.0), x)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_relative_position_invariance():
    x = small_inputs(1, 1, 20, 16, 16, seed=23)
    qh0, kh0 = R.angular_vectors(x["q"], x["k"], True, 10000.0, pos0=0)
    qh1, kh1 = R.angular_vectors(x["q"], x["k"], True, 10000.0, pos0=977)
    np.testing.assert_allclose(qh0 @ np.swapaxes(kh0, -1, -2), qh1 @ np.swapaxes(kh1, -1, -2),
                               atol=1e-12)


# ---------------------------------------------------------------- invariances

def test_causality():
    x = small_inputs(1, 2, 30, 8, 8, seed=31)
    o = R.causal_forward(**x)
    y = {key: np.array(val, copy=True) for key, val in x.items()}
    rng = np.random.default_rng(0)
    for key in ("q", "k", "v", "u"):
        y[key][..., 20:, :] = rng.normal(size=y[key][..., 20:, :].shape)
    y["g1"][..., 20:] += 1.0
    o2 = R.causal_forward(**y)
    np.testing.assert_array_equal(o[..., :20, :], o2[..., :20, :])


def test_linearity_scale_and_sign():
    x = small_inputs(1, 2, 30, 8, 8, seed=32)
    o = R.causal_forward(**x)
    y = dict(x)
    y["v"] = 2.5 * x["v"].astype(float) - 1.0 * np.roll(x["v"], 1, axis=-2)
    oy = R.causal_forward(**y)
    o_roll = R.causal_forward(**{**x, "v": np.roll(x["v"], 1, axis=-2)})
    assert rel(oy, 2.5 * o - o_roll) < TOL
    assert rel(R.causal_forward(**{**x, "q": 3.0 * x["q"].astype(float)}), o) < TOL
    assert rel(R.causal_forward(**{**x, "k": 0.25 * x["k"].astype(float)}), o) < TOL
    assert rel(R.causal_forward(**{**x, "q": -x["q"].astype(float)}), -o) < TOL


def test_lemma_norm_bound():
    """||o_t|| <= max_i ||v_i|| * sum_i |w_{t,i}| (|cos| <= 1)."""
    x = small_inputs(1, 2, 40, 8, 8, seed=33)
    o = R.causal_forward(**x)
    s = R.deviation_logits_causal(x["u"], x["mu"], x["tau"])
    W = R.explicit_weights_causal(s, x["g1"], x["gh"])
    vmax = np.max(np.linalg.norm(x["v"].astype(float), axis=-1), axis=-1)
    bound = vmax[..., None] * np.sum(np.abs(W), -1)
    assert np.all(np.linalg.norm(o, axis=-1) <= bound + 1e-14)


# ---------------------------------------------------------------- running max and stress

@pytest.mark.parametrize("scale", [10.0, 30.0])
def test_logit_stress_matches_explicit_weights(scale):
    x = small_inputs(1, 2, 48, 16, 16, seed=34, u_scale=scale)
    s = R.deviation_logits_causal(x["u"], x["mu"], x["tau"])
    assert s.max() - s.min() > 300.0 * (scale / 30.0)        # exp(s) alone would overflow/underflow
    o = R.causal_forward(**x)
    assert np.all(np.isfinite(o))
    assert rel(o, R.causal_brute_force(**x)) < 1e-11


# ---------------------------------------------------------------- decode continuity

@pytest.mark.parametrize("rope", [False, True])
def test_decode_continues_forward(rope):
    x = small_inputs(2, 2, 33, 16, 16, seed=35)
    o_full = R.causal_forward(**x, rope=rope)
    head = {key: (val[..., :32, :] if val.ndim == 4 else val[..., :32] if val.ndim == 3 else val)
            for key, val in x.items()}
    _, st = R.causal_forward(**head, rope=rope, return_state=True)
    tok = {key: (val[..., 32, :] if val.ndim == 4 else val[..., 32] if val.ndim == 3 else val)
           for key, val in x.items()}
    o_step, st2 = R.decode_step(st, tok["q"], tok["k"], tok["v"], tok["u"], x["mu"], x["tau"],
                                tok["g1"], tok["gh"], rope=rope)
    assert rel(o_step, o_full[..., 32, :]) < TOL
    assert np.all(st2["t"] == 33) and np.all(st["t"] == 32)


# ---------------------------------------------------------------- optional zero-order gate

def _gate0(x, seed):
    return np.random.default_rng(seed).normal(0.0, 1.5, size=x["g1"].shape)


def test_zero_order_gate_weight_rows_sum_to_sigma0():
    """With the zero-order term kept, row t of the weights sums to sigma0_t (1/t over t keys)."""
    x = small_inputs(2, 2, 30, 8, 8, seed=41)
    g0 = _gate0(x, 1)
    s = R.deviation_logits_causal(x["u"], x["mu"], x["tau"])
    W = R.explicit_weights_causal(s, x["g1"], x["gh"], g0)
    sig0 = 1.0 / (1.0 + np.exp(-g0))
    assert np.max(np.abs(W.sum(-1) - sig0)) < TOL
    assert np.all(np.triu(np.ones((30, 30)), 1)[None, None] * W == 0)
    We = R.explicit_weights_encoder(s, x["g1"], x["gh"], g0)
    assert np.max(np.abs(We.sum(-1) - sig0)) < TOL


def test_zero_order_gate_alone_is_causal_mean():
    """sigma1 = sigmah = 0, sigma0 = 1, q and k along one direction (cos = 1): o_t is the running
    mean of v_1..v_t, built here with a cumulative sum."""
    x = small_inputs(1, 2, 29, 8, 8, seed=42)
    x["k"] = np.broadcast_to(x["q"][:, :, :1, :], x["q"].shape).copy()
    x["q"] = 3.0 * x["k"]
    x["g1"] = np.full_like(x["g1"], -1000.0)
    x["gh"] = np.full_like(x["gh"], -1000.0)
    g0 = np.full(x["g1"].shape, 1000.0)
    v = x["v"].astype(float)
    ref = np.cumsum(v, axis=-2) / np.arange(1, 30)[:, None]
    assert rel(R.causal_forward(**x, g0=g0), ref) < TOL
    enc = R.encoder_forward(**x, g0=g0)
    assert rel(enc, np.broadcast_to(v.mean(axis=-2, keepdims=True), v.shape)) < TOL


@pytest.mark.parametrize("rope", [False, True])
def test_zero_order_gate_recurrence_matches_explicit_weights(rope):
    x = small_inputs(2, 3, 37, 16, 16, seed=43)
    g0 = _gate0(x, 2)
    o = R.causal_forward(**x, rope=rope, g0=g0)
    assert rel(o, R.causal_brute_force(**x, rope=rope, g0=g0)) < TOL
    assert rel(R.encoder_forward(**x, rope=rope, g0=g0), R.encoder_brute_force(**x, rope=rope, g0=g0)) < TOL
    # the term is additive: the difference to the gate-free output is sigma0_t/t sum_{i<=t} cos v
    cos = _cos(x, rope)
    N = cos.shape[-1]
    mask = np.tril(np.ones((N, N)))
    sig0 = 1.0 / (1.0 + np.exp(-g0))
    extra = ((cos * mask) @ x["v"].astype(float)) * (sig0 / np.arange(1, N + 1))[..., None]
    assert rel(o - R.causal_forward(**x, rope=rope), extra) < 1e-10


def test_zero_order_gate_decode_continues_forward():
    x = small_inputs(2, 2, 33, 16, 16, seed=44)
    g0 = _gate0(x, 3)
    o_full = R.causal_forward(**x, g0=g0)
    head = {key: (val[..., :32, :] if val.ndim == 4 else val[..., :32] if val.ndim == 3 else val)
            for key, val in x.items()}
    _, st = R.causal_forward(**head, return_state=True, g0=g0[..., :32])
    tok = {key: (val[..., 32, :] if val.ndim == 4 else val[..., 32] if val.ndim == 3 else val)
           for key, val in x.items()}
    o_step, _ = R.decode_step(st, tok["q"], tok["k"], tok["v"], tok["u"], x["mu"], x["tau"],
                              tok["g1"], tok["gh"], g0=g0[..., 32])
    assert rel(o_step, o_full[..., 32, :]) < TOL


@pytest.mark.parametrize("cut", [1, 17, 32])
def test_causal_forward_continues_from_state(cut):
    """causal_forward(state=...) over the rest of a sequence equals one pass over all of it, for
    the outputs and the final state (the continuation contract of the library's state_in)."""
    x = small_inputs(2, 2, 41, 16, 16, seed=45)
    g0 = _gate0(x, 4)
    o_full, st_full = R.causal_forward(**x, rope=True, g0=g0, return_state=True)
    head = {k: (v[..., :cut, :] if v.ndim == 4 else v[..., :cut] if v.ndim == 3 else v) for k, v in x.items()}
    tail = {k: (v[..., cut:, :] if v.ndim == 4 else v[..., cut:] if v.ndim == 3 else v) for k, v in x.items()}
    o1, st = R.causal_forward(**head, rope=True, g0=g0[..., :cut], return_state=True)
    o2, st2 = R.causal_forward(**tail, rope=True, g0=g0[..., cut:], state=st, return_state=True)
    assert rel(np.concatenate([o1, o2], axis=-2), o_full) < TOL
    for key in ("m", "E", "P", "Su", "F", "G", "H"):
        assert rel(st2[key], st_full[key]) < TOL, key
    assert np.all(st2["t"] == 41)


def test_zero_order_gate_first_token():
    """At t = 1 the zero-sum part vanishes and o_1 = sigma0_1 (q^_1 . k^_1) v_1."""
    x = small_inputs(2, 2, 1, 8, 8, seed=46)
    g0 = _gate0(x, 5)
    o = R.causal_forward(**x, g0=g0)
    sig0 = 1.0 / (1.0 + np.exp(-g0))
    ref = sig0[..., None] * _cos(x)[..., 0, 0][..., None, None] * x["v"].astype(float)
    assert rel(o, ref) < TOL


def test_encoder_single_token_is_zero_and_two_tokens_closed_form():
    """Encoder, N = 1: delta = 0 and softmax = 1, so every weight is zero. N = 2 with sigma1 = 1,
    sigmah = 0: w_{t,i} = (s_i - (s_1 + s_2)/2)/2, i.e. +-(s_2 - s_1)/4, the same for both queries."""
    x = small_inputs(2, 2, 1, 8, 8, seed=47)
    assert np.max(np.abs(R.encoder_forward(**x))) < 1e-12 * np.max(np.abs(x["v"]))
    x = small_inputs(1, 1, 2, 8, 8, seed=48)
    x["g1"] = np.full_like(x["g1"], 1000.0)
    x["gh"] = np.full_like(x["gh"], -1000.0)
    s = R.deviation_logits_encoder(x["u"], x["mu"], x["tau"])[0, 0]
    cos = _cos(x)[0, 0]
    v = x["v"][0, 0].astype(float)
    half = (s[1] - s[0]) / 4.0
    ref = np.stack([cos[t, 0] * (-half) * v[0] + cos[t, 1] * half * v[1] for t in range(2)])
    assert rel(R.encoder_forward(**x)[0, 0], ref) < TOL


def test_decode_from_empty_state_is_first_token():
    """One decode step from the empty state equals the causal forward of that one token (zero
    without the zero-order gate, sigma0 (q^.k^) v with it)."""
    x = small_inputs(2, 3, 1, 16, 16, seed=49)
    st = R.empty_state((2, 3), 16, 16)
    tok = {k: (v[..., 0, :] if v.ndim == 4 else v[..., 0] if v.ndim == 3 else v) for k, v in x.items()}
    g0 = _gate0(x, 6)
    o, st2 = R.decode_step(st, tok["q"], tok["k"], tok["v"], tok["u"], x["mu"], x["tau"], tok["g1"], tok["gh"],
                           g0=g0[..., 0])
    ref = R.causal_forward(**x, g0=g0)[..., 0, :]
    assert rel(o, ref) < TOL
    assert np.all(st2["t"] == 1)
