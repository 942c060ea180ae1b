"""Float64 CPU oracle for the ZeroS (zero-sum linear attention) forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the library's product path may import, call or execute
this module; only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP library and the library never falls back to it.

Sources (cited by page title and section; the pages are web summaries of arXiv 2602.05230):
  [Notes/zero-sum]  Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient
                    Transformers", section 关键设计, item "Softmax 零阶移除与零和权重构建":
                    softmax is split into a 1/t term, a first-order offset delta/t and a
                    higher-order residual eps; the 1/t term is dropped and the weight is
                    w_{t,i} = sigma1_t * delta_{t,i} / t + sigmah_t * eps_{t,i}, with sigmoid
                    gates that depend on the query step t. The weights sum to zero over i.
  [Notes/radial]    same page, item "径向-角向解耦": o_t = sum_{i<=t} r_{t,i} cos(theta) v_i
                    with cos(theta) the inner product of the L2-normalised q_t and k_i;
                    with RoPE the angular factor becomes q^_t R_{t-i} k^_i^T.
  [Notes/logits]    same page, item "偏差 logits 设计": s_i = -(1/sqrt(d)) u_i . ubar_i with
                    ubar_i = (e^tau mu + sum_{j<=i} u_j) / (e^tau + i).
  [Notes/scan]      same page, item "线性时间前缀扫描": the prefix states E, P, F, G, H and
                    o_t = q^_t (alpha_t F_t + beta_t G_t + gamma_t H_t).
  [Notes/training]  same page, section "损失函数 / 训练策略": causal (decoder) and
                    non-causal (encoder) modes.
  [Summary/plain]   ai.info page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers",
                    section "Methodology in Plain English" (same method in English).
  [Summary/SM]      same ai.info page and section: the same reweighting applied to standard
                    softmax attention gives the quadratic-time variant ZeroS-SM (also a row of the
                    MAD table in the Paper-Notes section 实验关键数据). Its exact form is in an
                    appendix the pages do not carry: parity unpinned against the authors.

Readings taken where the pages leave a step open (each is listed in the design notes):
  * delta_{t,i} = s_i - (1/t) sum_{j<=t} s_j, the first-order Taylor term of softmax about equal
    logits; eps_{t,i} = softmax_{t,i} - 1/t - delta_{t,i}/t.
  * Expanding w over the prefix sums gives w_{t,i} = alpha_t e^{s_i} + beta_t s_i + gamma_t with
    alpha_t = sigmah_t / E_t, beta_t = (sigma1_t - sigmah_t)/t,
    gamma_t = -(sigma1_t - sigmah_t) P_t / t^2 - sigmah_t / t  (see ``coefficients``).
  * Positions are 1-based in the formulas; the sum for ubar_i includes u_i; the causal sum over
    i <= t includes i = t.
  * The 1/sqrt(d) of the logit uses d_u, the length of the dot product.
  * mu (d_u vector) and tau (scalar) are per head; gates arrive as pre-activations and the
    logistic sigmoid is applied here.
  * L2 normalisation divides by max(||x||, 1e-12).
  * RoPE: interleaved pairs (2j, 2j+1), theta_j = base^(-2j/d), 0-based position p = t-1,
    applied after normalisation to both q^ and k^.
  * Encoder mode: one global prior-smoothed mean ubar over all N tokens, and every query uses
    the full-sequence sums with t replaced by N and its own gates.
  * Optional zero-order gate [Notes/zero-sum, design motivation; Summary/plain]: a first layer
    may keep the uniform term with its own step gate, w_{t,i} += sigma0_t / t (t = N in encoder
    mode); sigma0 = sigmoid(g0). Without g0 the term is absent (the default).
  * A running maximum m_t of the logits rescales e^{s}: the state stores
    Et = sum e^{s_i - m_t} and Ft = sum e^{s_i - m_t} k^_i^T v_i (this leaves o unchanged).
  * ZeroS-SM [Summary/SM]: the logits are the standard scaled dot products
    l_{t,i} = q_t . k_i / sqrt(d) (q and k as given, rotated by RoPE at their 0-based positions
    when asked; no normalisation and no separate cosine factor, the logits carry both); the row
    softmax over i <= t is split and reweighted exactly as above, w_{t,i} = sigma1_t delta_{t,i}/t
    + sigmah_t eps_{t,i} (+ sigma0_t / t), and o_t = sum_{i<=t} w_{t,i} v_i. Causal only.

Backward: ``causal_backward`` gives the gradients of L = <dO, o> for every input, by the chain
rule through the explicit weight definition (training replaces attention by this module
[Notes/training]); it is pinned by finite differences of the recurrent forward.

Array conventions: leading dimensions [B, H] (any number of leading dims works), then tokens,
then features. All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(x):
    return np.asarray(x, dtype=F64)


def sigmoid(x):
    """Logistic sigmoid, evaluated without overflow for large |x|."""
    x = _f64(x)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def l2_normalize(x):
    """Unit vectors along the last axis [Notes/radial]."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-12)


def rope_theta(d, base):
    """Per-pair frequencies theta_j = base^(-2j/d), j = 0 .. d/2-1."""
    j = np.arange(d // 2, dtype=F64)
    return np.power(F64(base), -2.0 * j / d)


def rope_rotate(x, positions, base):
    """Rotate interleaved pairs (2j, 2j+1) of x[..., n, d] by angle positions[n] * theta_j.

    [Notes/radial] (RoPE compatibility): q^_t R_t and k^_i R_i, so that their inner product
    depends on t - i only.
    """
    x = _f64(x)
    d = x.shape[-1]
    ang = _f64(positions)[:, None] * rope_theta(d, base)[None, :]      # [n, d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def angular_vectors(q, k, rope=False, rope_base=10000.0, pos0=0):
    """Return (q^, k^): L2-normalised and, optionally, RoPE-rotated at positions pos0 + 0..n-1."""
    qh, kh = l2_normalize(q), l2_normalize(k)
    if rope:
        pos = pos0 + np.arange(qh.shape[-2], dtype=F64)
        qh = rope_rotate(qh, pos, rope_base)
        kh = rope_rotate(kh, pos, rope_base)
    return qh, kh


def _prior(mu, tau):
    """(e^tau * mu, e^tau) with mu [..., d_u] and tau [...] broadcast to the leading dims."""
    et = np.exp(_f64(tau))
    return et[..., None] * _f64(mu), et


def deviation_logits_causal(u, mu, tau):
    """s_i = -(u_i . ubar_i)/sqrt(d_u), ubar_i = (e^tau mu + sum_{j<=i} u_j)/(e^tau + i).

    [Notes/logits]. u [..., N, d_u]; mu [..., d_u] and tau [...] broadcast over the leading
    dims (per head). Returns s [..., N].
    """
    u = _f64(u)
    N, du = u.shape[-2], u.shape[-1]
    emu, et = _prior(mu, tau)
    S = np.cumsum(u, axis=-2)
    i = np.arange(1, N + 1, dtype=F64)
    ubar = (emu[..., None, :] + S) / (et[..., None, None] + i[:, None])
    return -np.sum(u * ubar, axis=-1) / np.sqrt(F64(du))


def deviation_logits_encoder(u, mu, tau):
    """Encoder reading: one global ubar = (e^tau mu + sum_{all j} u_j)/(e^tau + N)."""
    u = _f64(u)
    N, du = u.shape[-2], u.shape[-1]
    emu, et = _prior(mu, tau)
    ubar = (emu + np.sum(u, axis=-2)) / (et[..., None] + N)
    return -np.einsum("...nc,...c->...n", u, ubar) / np.sqrt(F64(du))


def coefficients(t, Et, Pt, sig1, sigh, sig0=None):
    """alpha, beta, gamma of o_t = q^_t(alpha F + beta G + gamma H).

    Derivation from [Notes/zero-sum] with the readings above:
      w_{t,i} = sig1 (s_i - P_t/t)/t + sigh (e^{s_i}/E_t - 1/t - (s_i - P_t/t)/t)
              = (sigh/E_t) e^{s_i} + ((sig1 - sigh)/t) s_i + (-(sig1 - sigh) P_t/t^2 - sigh/t).
    Summing over i <= t gives alpha E_t + beta P_t + gamma t = 0 (the zero-sum property).
    ``Et`` may be the max-rescaled sum; alpha then multiplies the equally rescaled F.
    A zero-order gate adds the constant sig0/t to every w_{t,i}, that is to gamma.
    """
    t = _f64(t)
    d1 = _f64(sig1) - _f64(sigh)
    alpha = _f64(sigh) / _f64(Et)
    beta = d1 / t
    gamma = -d1 * _f64(Pt) / (t * t) - _f64(sigh) / t
    if sig0 is not None:
        gamma = gamma + _f64(sig0) / t
    return alpha, beta, gamma


# --------------------------------------------------------------------------------------------
# Recurrent (five-state) form: the oracle used at every size.
# --------------------------------------------------------------------------------------------

def empty_state(lead, d, d_u):
    """State before any token: t = 0, m = -inf, all sums zero. ``lead`` = leading shape."""
    lead = tuple(lead)
    return {
        "t": np.zeros(lead, dtype=np.int64),
        "m": np.full(lead, -np.inf, dtype=F64),
        "E": np.zeros(lead, dtype=F64),
        "P": np.zeros(lead, dtype=F64),
        "Su": np.zeros(lead + (d_u,), dtype=F64),
        "F": np.zeros(lead + (d, d), dtype=F64),
        "G": np.zeros(lead + (d, d), dtype=F64),
        "H": np.zeros(lead + (d, d), dtype=F64),
    }


def decode_step(state, q, k, v, u, mu, tau, g1, gh, rope=False, rope_base=10000.0, g0=None):
    """Advance the state by one token and return (o, new_state); ``state`` is not modified.

    q, k, v [..., d]; u [..., d_u]; mu [..., d_u]; tau, g1, gh (and g0) [...]. The token is at 1-based
    position t = state["t"] + 1 (RoPE position t - 1). States follow [Notes/scan]; the logit uses
    the running u-sum of [Notes/logits]; coefficients as in ``coefficients``.
    """
    st = {key: np.array(val, copy=True) for key, val in state.items()}
    o = _step_inplace(st, q, k, v, u, mu, tau, g1, gh, rope, rope_base, g0)
    return o, st


def _step_inplace(st, q, k, v, u, mu, tau, g1, gh, rope, rope_base, g0=None):
    t = st["t"] + 1
    tf = t.astype(F64)
    d_u = st["Su"].shape[-1]
    qh, kh = l2_normalize(q), l2_normalize(k)
    if rope:
        pos = (t - 1).astype(F64)
        qh, kh = _rope_per_item(qh, pos, rope_base), _rope_per_item(kh, pos, rope_base)
    u = _f64(u)
    emu, et = _prior(mu, tau)
    st["Su"] += u
    ubar = (emu + st["Su"]) / (et + tf)[..., None]
    s = -np.sum(u * ubar, axis=-1) / np.sqrt(F64(d_u))
    m_new = np.maximum(st["m"], s)
    with np.errstate(invalid="ignore"):
        c = np.exp(st["m"] - m_new)        # exp(-inf) = 0 for the empty state
    e = np.exp(s - m_new)
    st["E"] = c * st["E"] + e
    st["P"] = st["P"] + s
    kv = kh[..., :, None] * _f64(v)[..., None, :]
    F, G, H = st["F"], st["G"], st["H"]
    F *= c[..., None, None]
    F += e[..., None, None] * kv
    G += s[..., None, None] * kv
    H += kv
    st["m"] = m_new
    st["t"] = t
    a, b, g = coefficients(tf, st["E"], st["P"], sigmoid(g1), sigmoid(gh),
                           None if g0 is None else sigmoid(g0))
    M = a[..., None, None] * F + b[..., None, None] * G + g[..., None, None] * H
    return np.einsum("...j,...jm->...m", qh, M)


def _rope_per_item(x, pos, base):
    d = x.shape[-1]
    ang = pos[..., None] * rope_theta(d, base)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def causal_forward(q, k, v, u, mu, tau, g1, gh, rope=False, rope_base=10000.0,
                   return_state=False, state=None, g0=None):
    """Causal ZeroS forward as the sequential five-state recurrence (one step per token).

    q, k, v [..., N, d]; u [..., N, d_u]; mu [..., d_u] (per head, broadcast over batch);
    tau [...]; g1, gh [..., N]. Returns o [..., N, d] (float64), and the final state if asked.
    ``state`` continues from a previous state instead of the empty one. ``g0`` [..., N], if
    given, is the zero-order gate.
    """
    q, k, v, u = _f64(q), _f64(k), _f64(v), _f64(u)
    g1, gh = _f64(g1), _f64(gh)
    lead = q.shape[:-2]
    N, d = q.shape[-2], q.shape[-1]
    d_u = u.shape[-1]
    mu_b = np.broadcast_to(_f64(mu), lead + (d_u,))
    tau_b = np.broadcast_to(_f64(tau), lead)
    if state is None:
        st = empty_state(lead, d, d_u)
    else:
        st = {key: np.array(val, copy=True) for key, val in state.items()}
    o = np.empty(lead + (N, v.shape[-1]), dtype=F64)
    for n in range(N):
        o[..., n, :] = _step_inplace(st, q[..., n, :], k[..., n, :], v[..., n, :], u[..., n, :],
                                     mu_b, tau_b, g1[..., n], gh[..., n], rope, rope_base,
                                     None if g0 is None else _f64(g0)[..., n])
    return (o, st) if return_state else o


def encoder_forward(q, k, v, u, mu, tau, g1, gh, rope=False, rope_base=10000.0, g0=None):
    """Non-causal ZeroS forward [Notes/training]: every query uses the full-sequence sums.

    With t = N for every query: m = max s, E = sum e^{s-m}, P = sum s, F = sum e^{s-m} k^T v,
    G = sum s k^T v, H = sum k^T v, and o_t = q^_t(alpha_t F + beta_t G + gamma_t H) with the
    gates of token t.
    """
    v = _f64(v)
    qh, kh = angular_vectors(q, k, rope, rope_base)
    N = qh.shape[-2]
    s = deviation_logits_encoder(u, mu, tau)                          # [..., N]
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    E = np.sum(e, axis=-1)
    P = np.sum(s, axis=-1)
    F = np.einsum("...nj,...n,...nm->...jm", kh, e, v)
    G = np.einsum("...nj,...n,...nm->...jm", kh, s, v)
    H = np.einsum("...nj,...nm->...jm", kh, v)
    a, b, g = coefficients(F64(N), E[..., None], P[..., None], sigmoid(g1), sigmoid(gh),
                           None if g0 is None else sigmoid(g0))
    return (a[..., None] * (qh @ F) + b[..., None] * (qh @ G) + g[..., None] * (qh @ H))


# --------------------------------------------------------------------------------------------
# Explicit O(N^2) weights: the plain definition, used to pin the recurrence on small inputs.
# --------------------------------------------------------------------------------------------

def explicit_weights_causal(s, g1, gh, g0=None):
    """W[..., t, i] = w_{t,i} for i <= t, 0 above the diagonal [Notes/zero-sum].

    Row t (1-based) takes a softmax over s_1..s_t, its mean, delta = s_i - mean,
    eps = softmax - 1/t - delta/t, w = sigma1_t delta/t + sigmah_t eps (+ sigma0_t / t with a
    zero-order gate).
    """
    s = _f64(s)
    N = s.shape[-1]
    s1, sh = sigmoid(g1), sigmoid(gh)
    W = np.zeros(s.shape + (N,), dtype=F64)
    for ti in range(N):
        t = ti + 1
        row = s[..., :t]
        ex = np.exp(row - np.max(row, axis=-1, keepdims=True))
        sm = ex / np.sum(ex, axis=-1, keepdims=True)
        delta = row - np.mean(row, axis=-1, keepdims=True)
        eps = sm - 1.0 / t - delta / t
        W[..., ti, :t] = s1[..., ti, None] * delta / t + sh[..., ti, None] * eps
        if g0 is not None:
            W[..., ti, :t] += sigmoid(_f64(g0)[..., ti, None]) / t
    return W


def explicit_weights_encoder(s, g1, gh, g0=None):
    """Encoder weights: the same construction with the softmax and mean over all N tokens."""
    s = _f64(s)
    N = s.shape[-1]
    ex = np.exp(s - np.max(s, axis=-1, keepdims=True))
    sm = ex / np.sum(ex, axis=-1, keepdims=True)
    delta = s - np.mean(s, axis=-1, keepdims=True)
    eps = sm - 1.0 / N - delta / N
    s1, sh = sigmoid(g1)[..., :, None], sigmoid(gh)[..., :, None]
    W = s1 * delta[..., None, :] / N + sh * eps[..., None, :]
    if g0 is not None:
        W = W + sigmoid(_f64(g0))[..., :, None] / N
    return W


def causal_brute_force(q, k, v, u, mu, tau, g1, gh, rope=False, rope_base=10000.0, g0=None):
    """o_t = sum_{i<=t} w_{t,i} (q^_t . k^_i) v_i with the explicit weights [Notes/radial]."""
    qh, kh = angular_vectors(q, k, rope, rope_base)
    s = deviation_logits_causal(u, mu, tau)
    W = explicit_weights_causal(s, g1, gh, g0)
    cos = qh @ np.swapaxes(kh, -1, -2)
    return (W * cos) @ _f64(v)


def encoder_brute_force(q, k, v, u, mu, tau, g1, gh, rope=False, rope_base=10000.0, g0=None):
    qh, kh = angular_vectors(q, k, rope, rope_base)
    s = deviation_logits_encoder(u, mu, tau)
    W = explicit_weights_encoder(s, g1, gh, g0)
    cos = qh @ np.swapaxes(kh, -1, -2)
    return (W * cos) @ _f64(v)


# --------------------------------------------------------------------------------------------
# Backward pass: gradients of L = <dO, o> for the causal forward, by the chain rule through the
# explicit O(N^2) definition above (training uses the module in place of attention:
# [Notes/training]). Pinned by central finite differences of the recurrent ``causal_forward``.
# --------------------------------------------------------------------------------------------

def _unbroadcast(grad, shape):
    """Sum ``grad`` over the leading axes that broadcasting added to an input of ``shape``."""
    grad = _f64(grad)
    while grad.ndim > len(shape):
        grad = grad.sum(axis=0)
    for ax, n in enumerate(shape):
        if n == 1 and grad.shape[ax] != 1:
            grad = grad.sum(axis=ax, keepdims=True)
    return grad


def causal_backward(q, k, v, u, mu, tau, g1, gh, dO, rope=False, rope_base=10000.0, g0=None):
    """Gradients of L = sum_t dO_t . o_t through the causal forward.

    Shapes as in ``causal_forward``; dO [..., N, d]. Returns a dict with the gradients of q, k, v,
    u (the shapes of the inputs), mu and tau (summed over the dims they were broadcast over: the
    batch for per-head parameters), g1, gh and, when g0 is given, g0. Steps, in the order of the
    forward definition [Notes/zero-sum], [Notes/radial], [Notes/logits]:
      o = (W * C) v with C_{t,i} = q^_t . k^_i and the explicit weights W (i <= t);
      W_{t,i} = sigma1_t delta_{t,i}/t + sigmah_t eps_{t,i} (+ sigma0_t/t),
      delta_{t,i} = s_i - mean_{j<=t} s_j, eps = softmax_{t,i} - 1/t - delta/t;
      s_i = -(u_i . ubar_i)/sqrt(d_u), ubar_i = (e^tau mu + sum_{j<=i} u_j)/(e^tau + i);
      q^ = RoPE(q/|q|), k^ = RoPE(k/|k|).
    """
    q, k, v, u, dO = _f64(q), _f64(k), _f64(v), _f64(u), _f64(dO)
    lead = q.shape[:-2]
    N, d = q.shape[-2], q.shape[-1]
    du_dim = u.shape[-1]
    mu_in, tau_in = _f64(mu), _f64(tau)
    mu_b = np.broadcast_to(mu_in, lead + (du_dim,))
    tau_b = np.broadcast_to(tau_in, lead)
    tt = np.arange(1, N + 1, dtype=F64)                       # 1-based positions
    mask = np.tril(np.ones((N, N), dtype=bool))               # i <= t

    # ---- forward quantities of the explicit definition
    nq = np.maximum(np.sqrt(np.sum(q * q, axis=-1, keepdims=True)), 1e-12)
    nk = np.maximum(np.sqrt(np.sum(k * k, axis=-1, keepdims=True)), 1e-12)
    uq, uk = q / nq, k / nk                                   # unit vectors before RoPE
    pos = np.arange(N, dtype=F64)
    qh = rope_rotate(uq, pos, rope_base) if rope else uq
    kh = rope_rotate(uk, pos, rope_base) if rope else uk
    emu, et = _prior(mu_b, tau_b)
    S = np.cumsum(u, axis=-2)
    den = et[..., None] + tt                                  # e^tau + i
    ubar = (emu[..., None, :] + S) / den[..., None]
    s = -np.sum(u * ubar, axis=-1) / np.sqrt(F64(du_dim))
    sig1, sigh = sigmoid(g1), sigmoid(gh)
    sig0 = sigmoid(g0) if g0 is not None else None
    srow = np.where(mask, s[..., None, :], -np.inf)           # [..., t, i]
    ex = np.exp(srow - np.max(srow, axis=-1, keepdims=True))
    sm = ex / np.sum(ex, axis=-1, keepdims=True)              # softmax over i <= t (0 above)
    mean = np.cumsum(s, axis=-1) / tt                         # (1/t) sum_{j<=t} s_j
    delta = np.where(mask, s[..., None, :] - mean[..., :, None], 0.0)
    eps = np.where(mask, sm - 1.0 / tt[:, None] - delta / tt[:, None], 0.0)
    W = sig1[..., :, None] * delta / tt[:, None] + sigh[..., :, None] * eps
    if sig0 is not None:
        W = W + np.where(mask, sig0[..., :, None] / tt[:, None], 0.0)
    C = qh @ np.swapaxes(kh, -1, -2)

    # ---- o = (W * C) v
    Pm = W * C
    dv = np.swapaxes(Pm, -1, -2) @ dO
    dP = np.where(mask, dO @ np.swapaxes(v, -1, -2), 0.0)     # dO_t . v_i
    dW = dP * C
    dC = dP * W
    dqh = dC @ kh
    dkh = np.swapaxes(dC, -1, -2) @ qh

    # ---- W = sigma1 delta/t + sigmah eps (+ sigma0/t)
    dsig1 = np.sum(dW * delta, axis=-1) / tt
    dsigh = np.sum(dW * eps, axis=-1)
    dsig0 = np.sum(dW, axis=-1) / tt if sig0 is not None else None
    # eps = sm - 1/t - delta/t, so delta enters W with (sigma1 - sigmah)/t and sm with sigmah
    ddelta = dW * ((sig1 - sigh)[..., :, None] / tt[:, None])
    dsm = dW * sigh[..., :, None]
    # delta_{t,i} = s_i - (1/t) sum_{j<=t} s_j
    ds = np.sum(ddelta, axis=-2)
    rowsum = np.sum(ddelta, axis=-1)                          # [..., t]
    ds = ds - np.where(mask, (rowsum / tt)[..., :, None], 0.0).sum(axis=-2)
    # softmax Jacobian per row t: ds_j += sm_tj (dsm_tj - sum_i sm_ti dsm_ti)
    inner = np.sum(sm * dsm, axis=-1, keepdims=True)
    ds = ds + np.sum(sm * (dsm - inner), axis=-2)

    # ---- s = -(u . ubar)/sqrt(d_u), ubar_i = (e^tau mu + S_i)/(e^tau + i), S_i = sum_{j<=i} u_j
    rs = 1.0 / np.sqrt(F64(du_dim))
    du_ = -ubar * (ds * rs)[..., None]
    dubar = -u * (ds * rs)[..., None]
    dS = dubar / den[..., None]
    du_ = du_ + np.flip(np.cumsum(np.flip(dS, axis=-2), axis=-2), axis=-2)   # sum over i >= j
    dmu_full = et[..., None] * np.sum(dS, axis=-2)
    dtau_full = np.sum(np.sum(dubar * (mu_b[..., None, :] - ubar), axis=-1) * et[..., None] / den, axis=-1)

    # ---- q^ = RoPE(q/|q|): undo the rotation, then project out the radial direction
    if rope:
        dqh = rope_rotate(dqh, -pos, rope_base)
        dkh = rope_rotate(dkh, -pos, rope_base)
    dq = (dqh - uq * np.sum(uq * dqh, axis=-1, keepdims=True)) / nq
    dk = (dkh - uk * np.sum(uk * dkh, axis=-1, keepdims=True)) / nk

    out = {
        "q": dq, "k": dk, "v": dv, "u": du_,
        "mu": _unbroadcast(dmu_full, mu_in.shape), "tau": _unbroadcast(dtau_full, tau_in.shape),
        "g1": dsig1 * sig1 * (1.0 - sig1), "gh": dsigh * sigh * (1.0 - sigh),
    }
    if sig0 is not None:
        out["g0"] = dsig0 * sig0 * (1.0 - sig0)
    return out


# --------------------------------------------------------------------------------------------
# ZeroS-SM: the zero-sum reweighting applied to standard (quadratic) softmax attention.
# --------------------------------------------------------------------------------------------

def sm_logit_row(q, k, t, rope=False, rope_base=10000.0):
    """l_{t,i} = q_t . k_i / sqrt(d) for i = 1..t (1-based t) [Summary/SM]; with RoPE, q_t and
    k_i are rotated by their 0-based positions t - 1 and i - 1 first."""
    q, k = _f64(q), _f64(k)
    d = q.shape[-1]
    qt = q[..., t - 1:t, :]
    kr = k[..., :t, :]
    if rope:
        qt = rope_rotate(qt, np.array([t - 1], dtype=F64), rope_base)
        kr = rope_rotate(kr, np.arange(t, dtype=F64), rope_base)
    return np.sum(qt * kr, axis=-1) / np.sqrt(F64(d))              # [..., t]


def sm_weight_row(q, k, t, g1, gh, rope=False, rope_base=10000.0, g0=None):
    """Weights w_{t,1..t} of ZeroS-SM [Summary/SM] with the split of [Notes/zero-sum]: softmax
    p over the row, its first-order part dl = l - mean(l), the residual r = p - 1/t - dl/t, and
    w = sigma1_t dl / t + sigmah_t r (+ sigma0_t / t). g1, gh (g0) are the row's pre-activations."""
    lg = sm_logit_row(q, k, t, rope, rope_base)
    p = np.exp(lg - np.max(lg, axis=-1, keepdims=True))
    p = p / np.sum(p, axis=-1, keepdims=True)
    dl = lg - np.mean(lg, axis=-1, keepdims=True)
    r = p - 1.0 / t - dl / t
    w = sigmoid(g1)[..., None] * dl / t + sigmoid(gh)[..., None] * r
    if g0 is not None:
        w = w + sigmoid(g0)[..., None] / t
    return w


def sm_causal_forward(q, k, v, g1, gh, rope=False, rope_base=10000.0, g0=None, rows=None):
    """ZeroS-SM causal output o_t = sum_{i<=t} w_{t,i} v_i [Summary/SM], row by row.

    q, k, v [..., N, d]; g1, gh (g0) [..., N]. ``rows`` (1-based positions) limits the output to
    those rows, returned as [..., len(rows), d]; each row costs O(t d).
    """
    v = _f64(v)
    N = v.shape[-2]
    ts = range(1, N + 1) if rows is None else rows
    out = []
    for t in ts:
        w = sm_weight_row(q, k, t, _f64(g1)[..., t - 1], _f64(gh)[..., t - 1], rope, rope_base,
                          None if g0 is None else _f64(g0)[..., t - 1])
        out.append(np.einsum("...i,...id->...d", w, v[..., :t, :]))
    return np.stack(out, axis=-2)

