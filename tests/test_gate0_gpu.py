"""GPU parity of the optional zero-order gate (w_{t,i} += sigma0_t / t) on every path, through the
C ABI, against the float64 oracle on the same seeded inputs (bars as in the other parity tests:
relative L2 <= 1e-4 for float32, <= 2e-2 for bfloat16)."""
import numpy as np
import pytest
import torch

from oracle import zeros_ref as R
from synth import CONFIGS, make_inputs
from tests.gpu_helpers import TOL, rel_l2, slice_heads, tail_rel_l2, to_device, to_f64

pytestmark = pytest.mark.gpu

import zero_sum_attention_amd as Z  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _causal(t, rope, state_out=None, g0=True):
    return Z.zeros_fwd_causal(t["q"], t["k"], t["v"], t["u"], t["mu"], t["tau"], t["g1"], t["gh"],
                              g0=t["g0"] if g0 else None, rope=rope, state_out=state_out)


@pytest.mark.parametrize("d,N,dtype", [(16, 100, "f32"), (64, 33, "f32"), (128, 70, "f32"),
                                       (64, 129, "bf16"), (128, 300, "bf16"), (128, 1000, "bf16"),
                                       (32, 77, "bf16"), (64, 1, "bf16"), (16, 2, "f32")])
@pytest.mark.parametrize("rope", [False, True])
def test_causal_gate0(d, N, dtype, rope):
    """float32 path (any d) and the bfloat16 matrix-core path (d 64/128: several chunks, scan
    segments, ragged tails); the gate-free call on the same buffers still matches its oracle."""
    wl = CONFIGS[2].with_(B=2, H=3, N=N, d=d, d_u=d, dtype=dtype, seed=5000 + d + N)
    x = make_inputs(wl, gate0=True)
    t = to_device(x, dtype)
    o = to_f64(_causal(t, rope))
    ref = R.causal_forward(**x, rope=rope)
    assert rel_l2(o, ref) <= TOL[dtype]
    x0 = {k: v for k, v in x.items() if k != "g0"}
    o0 = to_f64(_causal(t, rope, g0=False))
    ref0 = R.causal_forward(**x0, rope=rope)
    if N == 1:
        assert np.max(np.abs(o0)) <= 1e-6     # one token and no zero-order term: exactly zero
    else:
        assert rel_l2(o0, ref0) <= TOL[dtype]
    assert rel_l2(o - o0, ref - ref0) <= 5 * TOL[dtype]


def test_causal_gate0_long_sampled_heads():
    """Long RoPE sequence at d 128 (64 scan segments of 2 chunks per head) with the gate on, sampled heads."""
    wl = CONFIGS[4].with_(B=1, H=4, N=8192, seed=5101)
    x = make_inputs(wl, gate0=True)
    t = to_device(x, wl.dtype)
    o = _causal(t, True)
    torch.cuda.synchronize()
    pairs = [(0, 0), (0, 3)]
    xs = slice_heads(x, pairs)
    ref = R.causal_forward(**xs, rope=True)
    got = np.stack([to_f64(o[b, h]) for b, h in pairs])[None]
    err, tail = rel_l2(got, ref), tail_rel_l2(got, ref, 1024)
    print(f"gate0 long rel_l2={err:.3e} tail(t>1024)={tail:.3e}", flush=True)
    assert err <= TOL["bf16"] and tail <= TOL["bf16"]


@pytest.mark.parametrize("d,N,dtype", [(16, 47, "f32"), (64, 197, "f32"), (64, 197, "bf16"),
                                       (128, 65, "bf16"), (64, 300, "bf16"), (128, 1000, "bf16"),
                                       (64, 1, "bf16"), (16, 2, "f32"), (128, 5000, "bf16")])
@pytest.mark.parametrize("rope", [False, True])
def test_encoder_gate0(d, N, dtype, rope):
    """Encoder: float32 path and both bfloat16 matrix-core variants (N <= 256 and longer)."""
    wl = CONFIGS[3].with_(B=2, H=3, N=N, d=d, d_u=d, dtype=dtype, seed=5200 + d + N)
    x = make_inputs(wl, gate0=True)
    t = to_device(x, dtype)
    o = Z.zeros_fwd_encoder(t["q"], t["k"], t["v"], t["u"], t["mu"], t["tau"], t["g1"], t["gh"],
                            g0=t["g0"], rope=rope)
    torch.cuda.synchronize()
    assert rel_l2(to_f64(o), R.encoder_forward(**x, rope=rope)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_gate0_continues_forward(dtype):
    """Prefill 64 tokens with the gate on (state_out), then one decode step with it."""
    wl = CONFIGS[2].with_(B=3, H=2, N=65, d=64, d_u=64, dtype=dtype, seed=5300)
    x = make_inputs(wl, gate0=True)
    cut = 64
    t = to_device(x, dtype)
    head = {k: (v[:, :, :cut].contiguous() if v.dim() >= 3 else v) for k, v in t.items()}
    st = Z.DecodeState(3, 2, 64, 64).reset()
    _causal(head, True, state_out=st)
    step = {k: (t[k][:, :, cut].contiguous()) for k in ("q", "k", "v", "u", "g1", "gh", "g0")}
    o_step = Z.zeros_decode_step(step["q"], step["k"], step["v"], step["u"], t["mu"], t["tau"],
                                 step["g1"], step["gh"], st, g0=step["g0"], rope=True)
    torch.cuda.synchronize()
    ref = R.causal_forward(**x, rope=True)[..., cut, :]
    assert rel_l2(to_f64(o_step), ref) <= TOL[dtype]
