"""Planted mistakes in the oracle are caught by its pins.

Each case below changes one step of the float64 oracle's source text (a dropped term, a wrong sign,
an index or scale off by one, a transposed operand), loads the changed module in place of
``oracle.zeros_ref`` in a fresh interpreter, and runs the oracle's pin tests
(``tests/test_oracle.py``: hand-worked fixtures, closed forms, the explicit O(N^2) weights,
library softmax limits, invariants; ``tests/test_oracle_backward.py``: finite differences of the
recurrent forward and the identities of the backward; ``tests/test_oracle_sm.py``: the ZeroS-SM
pins). Every planted mistake must make at least one pin fail. The
mutation is applied on the CPU, to a copy of the source in memory; nothing is written to disk.
Each original fragment must occur exactly once, so a case cannot silently stop applying when the
oracle's text changes.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "zeros_ref.py")

# (name, original fragment, planted mistake)
MUTATIONS = [
    ("gamma sign of the P term", "gamma = -d1 * _f64(Pt) / (t * t) - _f64(sigh) / t",
     "gamma = d1 * _f64(Pt) / (t * t) - _f64(sigh) / t"),
    ("gamma drops the uniform term", "gamma = -d1 * _f64(Pt) / (t * t) - _f64(sigh) / t",
     "gamma = -d1 * _f64(Pt) / (t * t)"),
    ("beta without 1/t", "    beta = d1 / t\n", "    beta = d1\n"),
    ("alpha without 1/E", "alpha = _f64(sigh) / _f64(Et)", "alpha = _f64(sigh)"),
    ("running mean counts i - 1 tokens",
     "ubar = (emu[..., None, :] + S) / (et[..., None, None] + i[:, None])",
     "ubar = (emu[..., None, :] + S) / (et[..., None, None] + i[:, None] - 1.0)"),
    ("running mean excludes u_i", "    S = np.cumsum(u, axis=-2)\n    i = np.arange",
     "    S = np.cumsum(u, axis=-2) - u\n    i = np.arange"),
    ("recurrent logit excludes u_i", '    st["Su"] += u\n    ubar = (emu + st["Su"]) / (et + tf)[..., None]\n',
     '    ubar = (emu + st["Su"]) / (et + tf)[..., None]\n    st["Su"] += u\n'),
    ("logit scale 1/d instead of 1/sqrt(d)", "return -np.sum(u * ubar, axis=-1) / np.sqrt(F64(du))",
     "return -np.sum(u * ubar, axis=-1) / F64(du)"),
    ("logit sign", "return -np.sum(u * ubar, axis=-1) / np.sqrt(F64(du))",
     "return np.sum(u * ubar, axis=-1) / np.sqrt(F64(du))"),
    ("prior without e^tau", "return et[..., None] * _f64(mu), et", "return _f64(mu), et"),
    ("norm squared", "n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))",
     "n = np.sum(x * x, axis=-1, keepdims=True)"),
    ("RoPE rotates the other way", "out[..., 0::2] = x0 * c - x1 * s\n    out[..., 1::2] = x0 * s + x1 * c",
     "out[..., 0::2] = x0 * c + x1 * s\n    out[..., 1::2] = -x0 * s + x1 * c"),
    ("RoPE frequencies over d/2", "return np.power(F64(base), -2.0 * j / d)",
     "return np.power(F64(base), -4.0 * j / d)"),
    ("F not rescaled when the maximum rises", "    F *= c[..., None, None]\n", ""),
    ("E not rescaled when the maximum rises", 'st["E"] = c * st["E"] + e', 'st["E"] = st["E"] + e'),
    ("G weighted by e^s", "    G += s[..., None, None] * kv\n", "    G += e[..., None, None] * kv\n"),
    ("transposed k^T v", "kv = kh[..., :, None] * _f64(v)[..., None, :]",
     "kv = _f64(v)[..., :, None] * kh[..., None, :]"),
    ("encoder uses N - 1", "a, b, g = coefficients(F64(N), E[..., None]",
     "a, b, g = coefficients(F64(N - 1), E[..., None]"),
    ("encoder drops the H state", "+ g[..., None] * (qh @ H))", ")"),
    ("delta without the mean", "delta = row - np.mean(row, axis=-1, keepdims=True)", "delta = row"),
    ("eps keeps the uniform term", "eps = sm - 1.0 / t - delta / t", "eps = sm - delta / t"),
    ("zero-order gate without 1/t", "gamma = gamma + _f64(sig0) / t", "gamma = gamma + _f64(sig0)"),
    # backward
    ("bwd: softmax Jacobian without its mean term", "ds = ds + np.sum(sm * (dsm - inner), axis=-2)",
     "ds = ds + np.sum(sm * dsm, axis=-2)"),
    ("bwd: delta without the row-mean term",
     "ds = ds - np.where(mask, (rowsum / tt)[..., :, None], 0.0).sum(axis=-2)", ""),
    ("bwd: delta scaled by sigma1 only", "ddelta = dW * ((sig1 - sigh)[..., :, None] / tt[:, None])",
     "ddelta = dW * (sig1[..., :, None] / tt[:, None])"),
    ("bwd: u misses the running-mean path",
     "du_ = du_ + np.flip(np.cumsum(np.flip(dS, axis=-2), axis=-2), axis=-2)", ""),
    ("bwd: running-mean path summed over i <= j", "du_ = du_ + np.flip(np.cumsum(np.flip(dS, axis=-2), axis=-2), axis=-2)",
     "du_ = du_ + np.cumsum(dS, axis=-2)"),
    ("bwd: mu without e^tau", "dmu_full = et[..., None] * np.sum(dS, axis=-2)", "dmu_full = np.sum(dS, axis=-2)"),
    ("bwd: tau sign", "dtau_full = np.sum(np.sum(dubar * (mu_b[..., None, :] - ubar)",
     "dtau_full = np.sum(np.sum(dubar * (ubar - mu_b[..., None, :])"),
    ("bwd: RoPE not undone", "        dqh = rope_rotate(dqh, -pos, rope_base)\n", ""),
    ("bwd: norm without the radial projection",
     "dq = (dqh - uq * np.sum(uq * dqh, axis=-1, keepdims=True)) / nq", "dq = dqh / nq"),
    ("bwd: v gradient uses W without the cosines", "dv = np.swapaxes(Pm, -1, -2) @ dO",
     "dv = np.swapaxes(W, -1, -2) @ dO"),
    ("bwd: k gradient from the untransposed product", "dkh = np.swapaxes(dC, -1, -2) @ qh", "dkh = dC @ qh"),
    ("bwd: sigmah gradient from delta", "dsigh = np.sum(dW * eps, axis=-1)", "dsigh = np.sum(dW * delta, axis=-1)"),
    ("bwd: gate derivative", '"g1": dsig1 * sig1 * (1.0 - sig1)', '"g1": dsig1 * sig1'),
    # ZeroS-SM
    ("SM: logits without 1/sqrt(d)", "return np.sum(qt * kr, axis=-1) / np.sqrt(F64(d))",
     "return np.sum(qt * kr, axis=-1)"),
    ("SM: residual keeps the uniform term", "r = p - 1.0 / t - dl / t", "r = p - dl / t"),
    ("SM: first order without the row mean", "dl = lg - np.mean(lg, axis=-1, keepdims=True)", "dl = lg"),
    ("SM: first-order term without 1/t", "w = sigmoid(g1)[..., None] * dl / t + sigmoid(gh)",
     "w = sigmoid(g1)[..., None] * dl + sigmoid(gh)"),
    ("SM: gates swapped", "w = sigmoid(g1)[..., None] * dl / t + sigmoid(gh)[..., None] * r",
     "w = sigmoid(gh)[..., None] * dl / t + sigmoid(g1)[..., None] * r"),
    ("SM: query rotated one position late", "qt = rope_rotate(qt, np.array([t - 1], dtype=F64), rope_base)",
     "qt = rope_rotate(qt, np.array([t], dtype=F64), rope_base)"),
    ("SM: zero-order gate without 1/t", "w = w + sigmoid(g0)[..., None] / t", "w = w + sigmoid(g0)[..., None]"),
    ("SM: softmax not normalised", "p = np.exp(lg - np.max(lg, axis=-1, keepdims=True))\n    p = p / np.sum(p, axis=-1, keepdims=True)",
     "p = np.exp(lg - np.max(lg, axis=-1, keepdims=True))"),
    ("bwd: zero-order gate without 1/t", "dsig0 = np.sum(dW, axis=-1) / tt if", "dsig0 = np.sum(dW, axis=-1) if"),
]

RUNNER = r"""
import sys, types
sys.path.insert(0, {root!r})
old, new = {old!r}, {new!r}
src = open({oracle!r}).read()
assert src.count(old) == 1, "fragment no longer unique in the oracle"
import oracle
mod = types.ModuleType("oracle.zeros_ref")
mod.__file__ = {oracle!r}
exec(compile(src.replace(old, new), {oracle!r}, "exec"), mod.__dict__)
sys.modules["oracle.zeros_ref"] = mod
oracle.zeros_ref = mod
import pytest
sys.exit(pytest.main([{tests!r}, {tests_bwd!r}, {tests_sm!r}, "-x", "-q", "-p", "no:cacheprovider", "-W", "ignore"]))
"""


def test_fragments_present():
    src = open(ORACLE).read()
    for name, old, _ in MUTATIONS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    code = RUNNER.format(root=ROOT, old=old, new=new, oracle=ORACLE,
                         tests=os.path.join(ROOT, "tests", "test_oracle.py"),
                         tests_bwd=os.path.join(ROOT, "tests", "test_oracle_backward.py"),
                         tests_sm=os.path.join(ROOT, "tests", "test_oracle_sm.py"))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert "fragment no longer unique" not in res.stderr, res.stderr[-2000:]
    # pytest exit code 1: a pin failed (the mistake was caught); 0 would mean every pin passed
    assert res.returncode == 1, f"planted mistake '{name}' passed every pin:\n{res.stdout[-2000:]}{res.stderr[-2000:]}"
