"""Pins of the float64 ZeroS-SM oracle (``sm_causal_forward``), independent of the HIP library.

ZeroS-SM is the zero-sum reweighting applied to standard softmax attention (ai.info page
"ZeroS: Zero-Sum Linear Attention for Efficient Transformers", Methodology in Plain English; the
split of the weight follows the Paper-Notes page, 关键设计). The pages give no formula of their
own for it, so these pins check the reading written in the oracle's header against a hand-worked
example, invariants and the special cases that reduce to textbook attention.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import zeros_ref as R

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _inputs(B=2, N=7, d=4, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    q = scale * rng.standard_normal((B, N, d))
    k, v = rng.standard_normal((B, N, d)), rng.standard_normal((B, N, d))
    g1, gh, g0 = (rng.standard_normal((B, N)) for _ in range(3))
    return q, k, v, g1, gh, g0


def test_hand_worked_t2():
    fx = json.load(open(os.path.join(GOLDEN, "sm_t2_hand.json")))
    x = {key: np.array(val, dtype=np.float64) for key, val in fx["inputs"].items()}
    o = R.sm_causal_forward(x["q"], x["k"], x["v"], x["g1"], x["gh"])
    np.testing.assert_allclose(o, np.array(fx["o"]), rtol=0, atol=fx["tol"])


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("with_g0", [False, True])
def test_rows_sum_to_the_zero_order_gate(rope, with_g0):
    q, k, _, g1, gh, g0 = _inputs(seed=3)
    for t in range(1, q.shape[-2] + 1):
        w = R.sm_weight_row(q, k, t, g1[:, t - 1], gh[:, t - 1], rope=rope,
                            g0=g0[:, t - 1] if with_g0 else None)
        want = R.sigmoid(g0[:, t - 1]) if with_g0 else np.zeros(q.shape[0])
        np.testing.assert_allclose(np.sum(w, axis=-1), want, atol=1e-13)


def test_saturated_gates_give_softmax_attention():
    """sigma1 = sigmah = sigma0 = 1: w = delta/t + eps + 1/t = softmax, standard causal attention."""
    q, k, v, _, _, _ = _inputs(N=9, d=6, seed=5)
    big = np.full(q.shape[:-1], 60.0)
    o = R.sm_causal_forward(q, k, v, big, big, g0=big)
    N, d = q.shape[-2], q.shape[-1]
    L = q @ np.swapaxes(k, -1, -2) / np.sqrt(d)
    L = np.where(np.tril(np.ones((N, N), dtype=bool)), L, -np.inf)
    np.testing.assert_allclose(o, softmax(L, axis=-1) @ v, rtol=1e-12, atol=1e-12)


def test_first_order_only_is_a_linear_attention():
    """sigmah = 0, sigma1 = 1: o_t = (1/t) sum_{i<=t} (l_ti - mean_t l) v_i, written with prefix
    sums of k v^T, k and v (the linear-time form)."""
    q, k, v, _, _, _ = _inputs(N=8, d=5, seed=7)
    N, d = q.shape[-2], q.shape[-1]
    o = R.sm_causal_forward(q, k, v, np.full(q.shape[:-1], 60.0), np.full(q.shape[:-1], -60.0))
    KV = np.cumsum(k[..., :, :, None] * v[..., :, None, :], axis=-3)     # sum_{i<=t} k_i v_i^T
    Ks, Vs = np.cumsum(k, axis=-2), np.cumsum(v, axis=-2)
    t = np.arange(1, N + 1, dtype=np.float64)
    lv = np.einsum("...tj,...tjm->...tm", q, KV) / np.sqrt(d)          # sum_i l_ti v_i
    lbar = np.sum(q * Ks, axis=-1) / (np.sqrt(d) * t)                   # mean_t l
    want = (lv - lbar[..., None] * Vs) / t[:, None]
    np.testing.assert_allclose(o, want, rtol=1e-11, atol=1e-12)


def test_residual_is_second_order():
    """sigma1 = 0, sigmah = 1: w = eps, the softmax residual above first order, which shrinks like
    the square of the logit scale."""
    outs = []
    for scale in (1e-2, 5e-3):
        q, k, v, _, _, _ = _inputs(N=6, d=4, seed=9, scale=scale)
        o = R.sm_causal_forward(q, k, v, np.full(q.shape[:-1], -60.0), np.full(q.shape[:-1], 60.0))
        outs.append(np.max(np.abs(o)))
    assert 3.6 < outs[0] / outs[1] < 4.4


@pytest.mark.parametrize("with_g0", [False, True])
def test_first_token(with_g0):
    q, k, v, g1, gh, g0 = _inputs(seed=11)
    o = R.sm_causal_forward(q, k, v, g1, gh, g0=g0 if with_g0 else None)
    want = R.sigmoid(g0[:, 0])[:, None] * v[:, 0] if with_g0 else np.zeros_like(v[:, 0])
    np.testing.assert_allclose(o[:, 0], want, atol=1e-14)


def test_rope_logits_depend_on_the_offset_only():
    """With RoPE, l_{t,i} = Re(sum_j z_q,j conj(z_k,j) e^{i (t - i) theta_j}) / sqrt(d) for the
    pairs read as complex numbers z = x_{2j} + i x_{2j+1}."""
    q, k, _, _, _, _ = _inputs(B=1, N=6, d=8, seed=13)
    d, base = 8, 10000.0
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    zq = q[..., 0::2] + 1j * q[..., 1::2]
    zk = k[..., 0::2] + 1j * k[..., 1::2]
    for t in range(1, 7):
        lg = R.sm_logit_row(q, k, t, rope=True, rope_base=base)
        for i in range(1, t + 1):
            want = np.real(np.sum(zq[0, t - 1] * np.conj(zk[0, i - 1]) * np.exp(1j * (t - i) * theta))) / np.sqrt(d)
            assert abs(lg[0, i - 1] - want) < 1e-12


def test_selected_rows_match_the_full_output():
    q, k, v, g1, gh, g0 = _inputs(N=9, seed=15)
    full = R.sm_causal_forward(q, k, v, g1, gh, rope=True, g0=g0)
    part = R.sm_causal_forward(q, k, v, g1, gh, rope=True, g0=g0, rows=[2, 5, 9])
    np.testing.assert_allclose(part, full[..., [1, 4, 8], :], rtol=0, atol=0)
