"""GPU parity of the causal backward (zeros_bwd_causal, through the C ABI) against the float64
oracle's gradients (``causal_backward``) on the same seeded inputs and upstream gradient.

Bars on the relative L2 error of each gradient tensor: 1e-4 for float32 inputs (float32
arithmetic throughout, as in the forward); for bfloat16 inputs the arithmetic is float32 too and
the only rounding beyond float32 is that of each gradient to bfloat16 on output (at most 2^-8
relative per element, about 1.7e-3 in RMS), so those are held to 5e-3 rather than the 2e-2 of
the forward's bfloat16 contract. dmu and dtau are float32 outputs on both paths: 1e-4.
"""
import numpy as np
import pytest
import torch

from oracle import zeros_ref as R
from synth import CONFIGS, make_inputs
from tests.gpu_helpers import rel_l2, to_device, to_f64

pytestmark = pytest.mark.gpu

import zero_sum_attention_amd as Z  # noqa: E402

BAR = {"f32": 1e-4, "bf16": 5e-3}
KEYS = ("q", "k", "v", "u", "mu", "tau", "g1", "gh")


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _check(x, dtype, rope, label, gate0=False):
    t = to_device(x, dtype)
    g = Z.zeros_bwd_causal(*(t[k] for k in KEYS), t["dO"], g0=t.get("g0"), rope=rope)
    torch.cuda.synchronize()
    args = {k: v for k, v in x.items() if k not in ("dO",)}
    ref = R.causal_backward(**args, dO=x["dO"], rope=rope)
    if x["q"].shape[-2] == 1 and "g0" not in x:
        # one token: o_1 = 0 for every input, so every gradient is exactly zero; float32 leaves
        # residues of a few ulp of the weight terms (|sigma| + |s_1| < 6) times |dO| |v| (< 36)
        for key, val in ref.items():
            assert np.all(val == 0.0)
            resid = float(np.max(np.abs(to_f64(g[key]))))
            print(f"bwd {label}: max|d{key}| = {resid:.1e}", flush=True)
            assert resid <= 1e-5, key
        return g
    errs = {}
    for key, val in ref.items():
        errs[key] = rel_l2(to_f64(g[key]), val)
    print(f"bwd {label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        bar = 1e-4 if key in ("mu", "tau") else BAR[dtype]
        assert e <= bar, (key, e)
    return g


def test_backward_config1_tiny():
    wl = CONFIGS[1]
    _check(make_inputs(wl, grad_out=True), wl.dtype, False, "config1")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("N", [1, 31, 33, 100])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rope", [False, True])
def test_backward_shapes(d, N, dtype, rope):
    """Every head dim, a single token, ragged tails around the 32-token scan chunk, both dtypes."""
    wl = CONFIGS[2].with_(B=2, H=2, N=N, d=d, d_u=d, dtype=dtype, seed=8000 + d + N)
    _check(make_inputs(wl, grad_out=True), dtype, rope, f"d={d} N={N} {dtype} rope={rope}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_zero_order_gate(dtype):
    wl = CONFIGS[2].with_(B=1, H=3, N=150, d=64, d_u=64, dtype=dtype, seed=8100)
    _check(make_inputs(wl, gate0=True, grad_out=True), dtype, True, f"gate0 {dtype}", gate0=True)


def test_backward_config2_lm_layer():
    """The LM-layer workload (B8 H8 N512 d64, float32), all 64 heads."""
    wl = CONFIGS[2]
    _check(make_inputs(wl, grad_out=True), wl.dtype, False, "config2")


def test_backward_bf16_d128_rope():
    """bfloat16 d 128 with RoPE, 1000 tokens: 32 scan chunks and a ragged tail."""
    wl = CONFIGS[4].with_(B=1, H=2, N=1000, seed=8200)
    _check(make_inputs(wl, grad_out=True), "bf16", True, "bf16 d128 rope N1000")


def test_backward_large_logits():
    """u x 10: the running maximum keeps every exponential of the reverse scans in range."""
    wl = CONFIGS[2].with_(B=1, H=2, N=300, d=32, d_u=32, dtype="f32", seed=8300)
    _check(make_inputs(wl, u_scale=10.0, grad_out=True), "f32", True, "u x 10")


def test_backward_deterministic_and_workspace_reuse():
    wl = CONFIGS[2].with_(B=2, H=2, N=200, d=64, d_u=64, dtype="f32", seed=8400)
    x = make_inputs(wl, grad_out=True)
    t = to_device(x, "f32")
    n = Z.zeros_bwd_causal_workspace_bytes(2, 2, 200, 64, 64, torch.float32)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    a = Z.zeros_bwd_causal(*(t[k] for k in KEYS), t["dO"], workspace=ws)
    b = Z.zeros_bwd_causal(*(t[k] for k in KEYS), t["dO"])
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_backward_empty_sequence():
    wl = CONFIGS[2].with_(B=1, H=2, N=0, d=16, d_u=16, seed=8500)
    t = to_device(make_inputs(wl, grad_out=True), "f32")
    g = Z.zeros_bwd_causal(*(t[k] for k in KEYS), t["dO"])
    torch.cuda.synchronize()
    assert torch.all(g["mu"] == 0) and torch.all(g["tau"] == 0)
