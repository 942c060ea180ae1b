"""Pins of the float64 backward oracle (``oracle.zeros_ref.causal_backward``).

The backward is the chain rule through the explicit O(N^2) weight definition. It is pinned to
things other than itself:
  * central finite differences of the *recurrent* forward ``causal_forward`` (a different
    implementation of the forward) along random directions, for every input;
  * identities the forward's form fixes: o is linear in v, so <dv, v> = <dO, o>; o does not change
    when one token's q or k is scaled by a positive factor, so dq_t . q_t = 0 and dk_i . k_i = 0
    for every token;
  * one token: o_1 = 0 for every input value, so every gradient is exactly zero;
  * causality: with dO zero after position T, the gradients equal those of the first T tokens
    and are zero for later tokens.
"""
import numpy as np
import pytest

from oracle import zeros_ref as R

KEYS = ("q", "k", "v", "u", "mu", "tau", "g1", "gh")


def _inputs(seed, B, H, N, d, u_scale=1.0, gate0=False):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.standard_normal((B, H, N, d)), k=rng.standard_normal((B, H, N, d)),
             v=rng.standard_normal((B, H, N, d)), u=u_scale * rng.standard_normal((B, H, N, d)),
             mu=0.1 * rng.standard_normal((H, d)), tau=rng.uniform(-1, 1, H),
             g1=rng.standard_normal((B, H, N)), gh=rng.standard_normal((B, H, N)))
    if gate0:
        x["g0"] = rng.standard_normal((B, H, N))
    return x, rng.standard_normal((B, H, N, d)), rng


def _loss(x, dO, rope, base):
    return float(np.sum(dO * R.causal_forward(**x, rope=rope, rope_base=base)))


@pytest.mark.parametrize("shape", [(1, 2, 9, 6), (2, 1, 17, 4), (1, 1, 2, 8), (1, 1, 33, 2)])
@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("gate0", [False, True])
def test_backward_matches_finite_differences(shape, rope, gate0):
    x, dO, rng = _inputs(sum(shape) + 10 * rope + 100 * gate0, *shape, gate0=gate0)
    base = 50.0
    g = R.causal_backward(**x, dO=dO, rope=rope, rope_base=base)
    # central differences in float64 carry a rounding floor of about eps |L| / h
    floor = 1e-10 * (1.0 + abs(_loss(x, dO, rope, base)))
    for key in x:
        dirn = rng.standard_normal(np.shape(x[key]))
        h = 1e-5
        xp, xm = dict(x), dict(x)
        xp[key] = x[key] + h * dirn
        xm[key] = x[key] - h * dirn
        fd = (_loss(xp, dO, rope, base) - _loss(xm, dO, rope, base)) / (2 * h)
        an = float(np.sum(g[key] * dirn))
        scale = np.linalg.norm(g[key]) * np.linalg.norm(dirn)
        assert abs(fd - an) <= 1e-7 * scale + floor, (key, fd, an)


def test_backward_large_logits_finite_differences():
    """u x 10: logits down to about -400, where only the running maximum keeps the forward finite."""
    x, dO, rng = _inputs(7, 1, 1, 24, 8, u_scale=10.0)
    g = R.causal_backward(**x, dO=dO)
    for key in ("u", "mu", "tau", "g1", "gh", "v"):
        dirn = rng.standard_normal(np.shape(x[key]))
        h = 1e-6
        xp, xm = dict(x), dict(x)
        xp[key] = x[key] + h * dirn
        xm[key] = x[key] - h * dirn
        fd = (_loss(xp, dO, False, 1e4) - _loss(xm, dO, False, 1e4)) / (2 * h)
        an = float(np.sum(g[key] * dirn))
        assert abs(fd - an) <= 1e-6 * np.linalg.norm(g[key]) * np.linalg.norm(dirn) + 1e-12, key


@pytest.mark.parametrize("rope", [False, True])
def test_backward_linearity_and_scale_identities(rope):
    x, dO, _ = _inputs(11, 2, 2, 40, 8, gate0=True)
    g = R.causal_backward(**x, dO=dO, rope=rope)
    o = R.causal_forward(**x, rope=rope)
    # o is linear in v
    assert abs(np.sum(g["v"] * x["v"]) - np.sum(dO * o)) <= 1e-12 * np.linalg.norm(dO) * np.linalg.norm(o) * 10
    # o is invariant to a positive scale of any single q_t or k_i
    for key in ("q", "k"):
        radial = np.sum(g[key] * x[key], axis=-1)
        assert np.max(np.abs(radial)) <= 1e-12 * np.max(np.linalg.norm(g[key], axis=-1) *
                                                        np.linalg.norm(x[key], axis=-1)) * 10, key


def test_backward_single_token_is_zero():
    """(Without the zero-order gate: with it the single weight is sigma0_1, not zero.)"""
    x, dO, _ = _inputs(12, 2, 3, 1, 8)
    g = R.causal_backward(**x, dO=dO, rope=True)
    for key, val in g.items():
        assert np.all(val == 0.0), key


@pytest.mark.parametrize("T", [1, 13, 31])
def test_backward_is_causal(T):
    x, dO, _ = _inputs(13, 1, 2, 32, 8)
    dO[..., T:, :] = 0.0
    g = R.causal_backward(**x, dO=dO, rope=True)
    xs = {k: (v[..., :T, :] if k in ("q", "k", "v", "u") else v[..., :T] if k in ("g1", "gh") else v)
          for k, v in x.items()}
    gs = R.causal_backward(**xs, dO=dO[..., :T, :], rope=True)
    for key in ("q", "k", "v", "u"):
        assert np.allclose(g[key][..., :T, :], gs[key], rtol=0, atol=1e-12), key
        assert np.all(g[key][..., T:, :] == 0.0), key
    for key in ("g1", "gh"):
        assert np.allclose(g[key][..., :T], gs[key], rtol=0, atol=1e-12), key
        assert np.all(g[key][..., T:] == 0.0), key
    for key in ("mu", "tau"):
        assert np.allclose(g[key], gs[key], rtol=0, atol=1e-12), key
