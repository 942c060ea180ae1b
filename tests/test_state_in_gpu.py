"""GPU parity of the causal forward continued from a state (chunked prefill), through the C ABI,
against the float64 oracle run over the whole sequence in one pass (bars as in the other parity
tests: relative L2 <= 1e-4 for float32, <= 2e-2 for bfloat16; the final state's float32 scalars to
1e-5, its matrices to 1e-5 on the float32 path and to the bfloat16-operand bar on the matrix-core
path)."""
import numpy as np
import pytest
import torch

from oracle import zeros_ref as R
from synth import CONFIGS, make_inputs
from tests.gpu_helpers import SCALAR_STATE_TOL, TOL, rel_l2, state_matrix_tol, to_device, to_f64

pytestmark = pytest.mark.gpu

import zero_sum_attention_amd as Z  # noqa: E402

TOKEN_KEYS = ("q", "k", "v", "u", "g1", "gh", "g0")


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def _part(t, a, b):
    """Tokens [a, b) of every token tensor (mu, tau unchanged)."""
    return {k: (v[:, :, a:b].contiguous() if k in TOKEN_KEYS else v) for k, v in t.items()}


def _causal(t, rope, state_in=None, state_out=None):
    return Z.zeros_fwd_causal(t["q"], t["k"], t["v"], t["u"], t["mu"], t["tau"], t["g1"], t["gh"],
                              g0=t.get("g0"), rope=rope, state_in=state_in, state_out=state_out)


def _check_state(got, ref, dtype, d):
    """Scalars (m, E, P, S_u) to 1e-5 on every path; F, G, H to the bar of the path that ran."""
    for key in ("m", "E", "P", "Su"):
        assert rel_l2(got[key], ref[key]) <= SCALAR_STATE_TOL, key
    bar = state_matrix_tol(dtype, d)
    errs = {key: rel_l2(got[key], ref[key]) for key in ("F", "G", "H")}
    print(f"state {dtype} d={d} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" (bar {bar:g})",
          flush=True)
    for key, e in errs.items():
        assert e <= bar, key


def _state_np(st):
    return {"F": to_f64(st.F), "G": to_f64(st.G), "H": to_f64(st.Hs), "Su": to_f64(st.Su),
            "m": to_f64(st.m), "E": to_f64(st.E), "P": to_f64(st.P),
            "t": st.t.cpu().numpy().astype(np.int64)}


@pytest.mark.parametrize("d,dtype,cut,N", [(16, "f32", 37, 100), (64, "f32", 64, 130), (32, "f32", 1, 40),
                                           (64, "bf16", 70, 200), (128, "bf16", 129, 300)])
@pytest.mark.parametrize("rope", [False, True])
def test_continuation_matches_one_pass(d, dtype, cut, N, rope):
    """Prefix [0, cut) with state_out, then [cut, N) from it: the outputs and the final state
    equal the oracle's single pass. bfloat16 d 64/128 calls (prefix and continuation) run on the
    matrix-core path, the continuation over several scan segments."""
    wl = CONFIGS[2].with_(B=2, H=3, N=N, d=d, d_u=d, dtype=dtype, seed=6000 + d + cut)
    x = make_inputs(wl, gate0=(d == 64))
    t = to_device(x, dtype)
    a = Z.DecodeState(2, 3, d, d).reset()
    b = Z.DecodeState(2, 3, d, d).reset()
    o1 = _causal(_part(t, 0, cut), rope, state_out=a)
    o2 = _causal(_part(t, cut, N), rope, state_in=a, state_out=b)
    torch.cuda.synchronize()
    o = np.concatenate([to_f64(o1), to_f64(o2)], axis=2)
    ref, st = R.causal_forward(**x, rope=rope, return_state=True)
    assert rel_l2(o[:, :, cut:], ref[:, :, cut:]) <= TOL[dtype]
    assert rel_l2(o, ref) <= TOL[dtype]
    got = _state_np(b)
    assert np.all(got["t"] == N)
    _check_state(got, st, dtype, d)


@pytest.mark.parametrize("d,dtype", [(32, "f32"), (64, "bf16"), (128, "bf16")])
def test_continuation_heads_at_different_positions(d, dtype):
    """Batch 0 continues after 40 tokens, batch 1 after 75 (one state assembled from two
    prefills); each continues for 50 tokens in one call (bfloat16 d 64/128: the matrix-core
    path with a per-head position offset)."""
    wl = CONFIGS[2].with_(B=2, H=2, N=125, d=d, d_u=d, dtype=dtype, seed=6100 + d)
    x = make_inputs(wl)
    t = to_device(x, dtype)
    s40 = Z.DecodeState(2, 2, d, d).reset()
    s75 = Z.DecodeState(2, 2, d, d).reset()
    _causal(_part(t, 0, 40), True, state_out=s40)
    _causal(_part(t, 0, 75), True, state_out=s75)
    a = Z.DecodeState(2, 2, d, d).reset()
    for name in ("F", "G", "Hs", "Su", "m", "E", "P", "t"):
        getattr(a, name)[0].copy_(getattr(s40, name)[0])
        getattr(a, name)[1].copy_(getattr(s75, name)[1])
    cont = {k: (torch.stack([v[0, :, 40:90], v[1, :, 75:125]]).contiguous() if k in TOKEN_KEYS else v)
            for k, v in t.items()}
    b = Z.DecodeState(2, 2, d, d).reset()
    o = to_f64(_causal(cont, True, state_in=a, state_out=b))
    ref0 = R.causal_forward(**{k: (v[:1, :, :90] if k in TOKEN_KEYS else v) for k, v in x.items()}, rope=True)
    ref1 = R.causal_forward(**{k: (v[1:, :, :125] if k in TOKEN_KEYS else v) for k, v in x.items()}, rope=True)
    assert rel_l2(o[:1], ref0[:, :, 40:]) <= TOL[dtype]
    assert rel_l2(o[1:], ref1[:, :, 75:]) <= TOL[dtype]
    tt = b.t.cpu().numpy()
    assert np.all(tt[0] == 90) and np.all(tt[1] == 125)


def test_continuation_long_bf16_prefix():
    """A 4096-token bf16 d 128 RoPE prefix, then 1000 more tokens (16 scan segments of one chunk:
    the combine starts from the given state)."""
    wl = CONFIGS[4].with_(B=1, H=2, N=5096, seed=6200)
    x = make_inputs(wl)
    t = to_device(x, wl.dtype)
    a = Z.DecodeState(1, 2, 128, 128).reset()
    _causal(_part(t, 0, 4096), True, state_out=a)
    o = to_f64(_causal(_part(t, 4096, 5096), True, state_in=a))
    ref = R.causal_forward(**x, rope=True)[:, :, 4096:]
    err = rel_l2(o, ref)
    print(f"continuation after 4096 tokens rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_continuation_empty_call_copies_state():
    d = 16
    wl = CONFIGS[2].with_(B=1, H=2, N=30, d=d, d_u=d, dtype="f32", seed=6300)
    t = to_device(make_inputs(wl), "f32")
    a = Z.DecodeState(1, 2, d, d).reset()
    _causal(t, False, state_out=a)
    b = Z.DecodeState(1, 2, d, d).reset()
    _causal(_part(t, 30, 30), False, state_in=a, state_out=b)
    torch.cuda.synchronize()
    for name in ("F", "G", "Hs", "Su", "m", "E", "P", "t"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


@pytest.mark.parametrize("d,dtype", [(16, "f32"), (128, "bf16")])
def test_continuation_from_empty_state(d, dtype):
    """state_in at t = 0 (a reset state) gives the plain forward and its final state."""
    wl = CONFIGS[2].with_(B=2, H=2, N=150, d=d, d_u=d, dtype=dtype, seed=6400 + d)
    x = make_inputs(wl)
    t = to_device(x, dtype)
    a = Z.DecodeState(2, 2, d, d).reset()
    b = Z.DecodeState(2, 2, d, d).reset()
    o = to_f64(_causal(t, True, state_in=a, state_out=b))
    ref, st = R.causal_forward(**x, rope=True, return_state=True)
    assert rel_l2(o, ref) <= TOL[dtype]
    got = _state_np(b)
    assert np.all(got["t"] == 150)
    _check_state(got, st, dtype, d)


# ------------------------------------------------------------------ segmented float32 scan

@pytest.mark.parametrize("d,N,dtype,B,H", [(64, 1000, "f32", 1, 2), (16, 777, "f32", 2, 1), (128, 700, "f32", 1, 1),
                                           (32, 900, "bf16", 1, 2)])
@pytest.mark.parametrize("rope", [False, True])
def test_float32_path_segments(d, N, dtype, B, H, rope):
    """Sequences long enough for the float32 path to split each head into scan segments (pass 1,
    combine, main): outputs and final state against the oracle; the same again continued from a
    state after 320 tokens."""
    wl = CONFIGS[2].with_(B=B, H=H, N=N, d=d, d_u=d, dtype=dtype, seed=6500 + d + N)
    x = make_inputs(wl, gate0=(d == 16))
    t = to_device(x, dtype)
    st = Z.DecodeState(B, H, d, d).reset()
    o = to_f64(_causal(t, rope, state_out=st))
    ref, sref = R.causal_forward(**x, rope=rope, return_state=True)
    err = rel_l2(o, ref)
    print(f"segmented float32 path d={d} N={N} rel_l2={err:.3e}", flush=True)
    assert err <= TOL[dtype]
    got = _state_np(st)
    _check_state(got, sref, dtype, d)
    a = Z.DecodeState(B, H, d, d).reset()
    _causal(_part(t, 0, 320), rope, state_out=a)
    o2 = to_f64(_causal(_part(t, 320, N), rope, state_in=a))
    assert rel_l2(o2, ref[:, :, 320:]) <= TOL[dtype]


@pytest.mark.parametrize("B,H,N,d", [(1, 3, 577, 32), (1, 1, 255, 16), (1, 1, 257, 16), (3, 1, 1000, 128),
                                     (1, 1, 4097, 64)])
def test_float32_segment_boundaries(B, H, N, d):
    """Segment plans with a one-token last segment (577 tokens, 3 heads), two segments of 127/128
    and 129/128 tokens, an odd head count (no XCD regrouping), and 22 segments (three combine
    batches); outputs against the oracle."""
    wl = CONFIGS[2].with_(B=B, H=H, N=N, d=d, d_u=d, dtype="f32", seed=6600 + N + d)
    x = make_inputs(wl)
    t = to_device(x, "f32")
    o = to_f64(_causal(t, True))
    err = rel_l2(o, R.causal_forward(**x, rope=True))
    print(f"f32 segments B{B} H{H} N{N} d{d} rel_l2={err:.3e}", flush=True)
    assert err <= TOL["f32"]


def test_empty_bf16_call_writes_empty_state():
    """N = 0 on the bfloat16 d 128 shape: without state_in the (matrix-core) call writes the empty
    state; with state_in it copies that state."""
    wl = CONFIGS[4].with_(B=1, H=2, N=40, seed=6700)
    t = to_device(make_inputs(wl), wl.dtype)
    a = Z.DecodeState(1, 2, 128, 128)
    for name in ("F", "G", "Hs", "Su", "m", "E", "P"):
        getattr(a, name).fill_(7.0)
    a.t.fill_(5)
    _causal(_part(t, 0, 0), True, state_out=a)
    torch.cuda.synchronize()
    for name in ("F", "G", "Hs", "Su", "E", "P"):
        assert torch.all(getattr(a, name) == 0), name
    assert torch.all(a.t == 0) and torch.all(torch.isneginf(a.m))
    b = Z.DecodeState(1, 2, 128, 128).reset()
    _causal(_part(t, 0, 40), True, state_out=b)
    c = Z.DecodeState(1, 2, 128, 128)
    _causal(_part(t, 40, 40), True, state_in=b, state_out=c)
    torch.cuda.synchronize()
    for name in ("F", "G", "Hs", "Su", "m", "E", "P", "t"):
        assert torch.equal(getattr(b, name), getattr(c, name)), name
