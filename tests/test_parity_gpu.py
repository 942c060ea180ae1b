"""GPU parity: libzeros (through its C ABI) against the float64 oracle on the same seeded inputs.

Bar: relative L2 error of the whole output <= 1e-4 for float32 inputs and <= 2e-2 for bfloat16
inputs with float32 accumulation. Sizes span several 32-token chunks and a ragged tail; the
full-size workloads are compared on sampled heads, which the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

from oracle import zeros_ref as R
from synth import CONFIGS, make_inputs
from synth.inputs import decode_prefill_batch
from tests.gpu_helpers import (SCALAR_STATE_TOL, STATE_TOL_BF16, TOL, rel_l2, row_rel_p99, slice_heads,
                               tail_rel_l2, to_device, to_f64)

pytestmark = pytest.mark.gpu

# Where the exact output is zero (a single token, u = 0) float32 rounding leaves residues of
# order eps32 * |v|: bound them absolutely.
ZERO_ABS = 1e-6
# The same on the bfloat16 matrix-core path: the weight of the single key of row 1 is formed in
# float32 as sigmah*1 + (sigma1 - sigmah) s_1 - (sigma1 - sigmah) s_1 - sigmah (exactly 0), which
# leaves |w| <= a few ulp of (|sigma| + |s_1|) < 6, i.e. below 4 * 6 * 2^-24 = 1.5e-6; rounding w to
# bfloat16 keeps it that small, |q^ . k^| <= 1 and |v| < 6 for N(0,1) rows of 128 features, and
# the bfloat16 output rounding is relative, so |o_1| < 1e-5.
ZERO_ABS_MFMA = 1e-5

import zero_sum_attention_amd as Z  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def run_causal(x, dtype, rope=False, state_out=None):
    t = to_device(x, dtype)
    o = Z.zeros_fwd_causal(t["q"], t["k"], t["v"], t["u"], t["mu"], t["tau"], t["g1"], t["gh"],
                           rope=rope, state_out=state_out)
    torch.cuda.synchronize()
    return o


def run_encoder(x, dtype, rope=False):
    t = to_device(x, dtype)
    o = Z.zeros_fwd_encoder(t["q"], t["k"], t["v"], t["u"], t["mu"], t["tau"], t["g1"], t["gh"], rope=rope)
    torch.cuda.synchronize()
    return o


def test_library_is_native():
    lib = Z.load_library()
    assert lib.zeros_abi_version() == 4
    assert torch.cuda.is_available()


# ------------------------------------------------------------------ the configured workloads

def test_config1_tiny_causal():
    wl = CONFIGS[1]
    x = make_inputs(wl)
    o = to_f64(run_causal(x, wl.dtype))
    ref = R.causal_forward(**x)
    assert rel_l2(o, ref) <= TOL["f32"]
    assert rel_l2(o, R.causal_brute_force(**x)) <= TOL["f32"]


def test_config2_lm_layer_causal():
    wl = CONFIGS[2]
    x = make_inputs(wl)
    o = to_f64(run_causal(x, wl.dtype))
    ref = R.causal_forward(**x)
    err = rel_l2(o, ref)
    print(f"config2 rel_l2={err:.3e}", flush=True)
    assert err <= TOL["f32"]


def test_config3_vit_encoder():
    wl = CONFIGS[3]
    x = make_inputs(wl)
    o = to_f64(run_encoder(x, wl.dtype))
    ref = R.encoder_forward(**x)
    err = rel_l2(o, ref)
    print(f"config3 rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_config4_long_rope_sampled_heads():
    wl = CONFIGS[4]
    x = make_inputs(wl)
    o = run_causal(x, wl.dtype, rope=True)
    pairs = [(0, 0), (1, 15), (0, 9)]
    xs = slice_heads(x, pairs)
    ref = R.causal_forward(**xs, rope=True)
    got = np.stack([to_f64(o[b, h]) for b, h in pairs])[None]
    err, tail = rel_l2(got, ref), tail_rel_l2(got, ref, 1024)
    p99 = row_rel_p99(got, ref, 1e-3)
    print(f"config4 sampled rel_l2={err:.3e} tail(t>1024)={tail:.3e} row_p99={p99:.3e}", flush=True)
    assert err <= TOL["bf16"]
    # the late rows: the tail bar of the long-sequence test, and 3x the per-row p99 measured on
    # correct builds (1.1e-2); a chunk computed from another chunk's v shows ~1e-1
    assert tail <= 6e-3
    assert p99 <= 3e-2
    assert np.all(np.isfinite(to_f64(o)))


def test_config4_repeat_bitwise():
    """The full-size call twice on the same inputs and workspace gives the same bits: every
    reduction order is fixed, so a difference can only come from a read racing a write (such as a
    direct copy into LDS not yet landed), which a full-size run under load exposes."""
    wl = CONFIGS[4]
    t = to_device(make_inputs(wl), wl.dtype)
    ws = torch.empty(Z.zeros_fwd_causal_workspace_bytes(wl.B, wl.H, wl.N, wl.d, wl.d_u, torch.bfloat16, True),
                     dtype=torch.uint8, device=t["q"].device)
    outs = []
    for _ in range(3):
        o = Z.zeros_fwd_causal(t["q"], t["k"], t["v"], t["u"], t["mu"], t["tau"], t["g1"], t["gh"], rope=True,
                               workspace=ws)
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


# ------------------------------------------------------------------ shapes, tails, options

@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("N", [1, 31, 33, 100])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rope", [False, True])
def test_causal_shapes(d, N, dtype, rope):
    wl = CONFIGS[2].with_(B=2, H=3, N=N, d=d, d_u=d, dtype=dtype, seed=1000 + d + N)
    x = make_inputs(wl)
    o = to_f64(run_causal(x, dtype, rope=rope))
    ref = R.causal_forward(**x, rope=rope)
    assert np.max(np.abs(o[..., 0, :])) <= ZERO_ABS      # o_1 = 0
    if N > 1:
        assert rel_l2(o, ref) <= TOL[dtype]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [64, 65, 129, 300, 1000])
@pytest.mark.parametrize("rope", [False, True])
def test_causal_mfma_chunks(d, N, rope):
    """bfloat16 d in {64, 128} runs on the matrix-core path: several 64-token chunks, ragged tails."""
    wl = CONFIGS[4].with_(B=2, H=2, N=N, d=d, d_u=d, seed=3000 + d + N)
    x = make_inputs(wl)
    o = to_f64(run_causal(x, "bf16", rope=rope))
    ref = R.causal_forward(**x, rope=rope)
    err = rel_l2(o, ref)
    print(f"mfma d={d} N={N} rope={rope} rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    o1 = float(np.max(np.abs(o[..., 0, :])))
    print(f"mfma d={d} N={N} rope={rope} max|o_1|={o1:.2e}", flush=True)
    assert o1 <= ZERO_ABS_MFMA


@pytest.mark.parametrize("rope", [False, True])
def test_causal_mfma_state_out(rope):
    wl = CONFIGS[4].with_(B=2, H=2, N=333, seed=3100)
    x = make_inputs(wl)
    st = Z.DecodeState(2, 2, 128, 128).reset()
    run_causal(x, "bf16", rope=rope, state_out=st)
    _, ref = R.causal_forward(**x, rope=rope, return_state=True)
    got = _state_np(st)
    assert np.all(got["t"] == 333)
    for key in ("m", "E", "P", "Su"):
        assert rel_l2(got[key], ref[key]) <= SCALAR_STATE_TOL, key
    errs = {key: rel_l2(got[key], ref[key]) for key in ("F", "G", "H")}
    print("mfma state_out " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= STATE_TOL_BF16, key


@pytest.mark.parametrize("d", [64, 128])
def test_causal_segments_ragged_sampled_heads(d):
    """32 heads, N = 3000: 47 chunks cut into 8 scan segments of 6 chunks (the last one 5 chunks,
    its last chunk 56 tokens), chained by pass 1 and the segment combine; outputs and the final
    recurrent state of sampled heads against the oracle."""
    wl = CONFIGS[4].with_(B=2, H=16, N=3000, d=d, d_u=d, seed=3300 + d)
    x = make_inputs(wl)
    st = Z.DecodeState(2, 16, d, d).reset()
    o = run_causal(x, "bf16", rope=True, state_out=st)
    pairs = [(0, 0), (1, 7), (0, 15)]
    xs = slice_heads(x, pairs)
    ref, ref_st = R.causal_forward(**xs, rope=True, return_state=True)
    got = np.stack([to_f64(o[b, h]) for b, h in pairs])[None]
    err = rel_l2(got, ref)
    print(f"segments d={d} N=3000 sampled rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    gst = _state_np(st)
    for key in ("m", "E", "P", "Su"):
        g = np.stack([gst[key][b, h] for b, h in pairs])[None]
        assert rel_l2(g, ref_st[key]) <= SCALAR_STATE_TOL, key
    for key in ("F", "G", "H"):
        g = np.stack([gst[key][b, h] for b, h in pairs])[None]
        e = rel_l2(g, ref_st[key])
        print(f"segments d={d} state {key}={e:.2e}", flush=True)
        assert e <= STATE_TOL_BF16, key


@pytest.mark.parametrize("scale", [10.0, 30.0])
def test_causal_segments_large_logits(scale):
    """bfloat16 scan path with logits scaled up so that the running maximum jumps by many nats
    between chunks: the chunk factors rX come out tiny or zero, which the scan's scaled state basis
    has to absorb (fold into the state, floor of the factor) across chained segments."""
    wl = CONFIGS[4].with_(B=2, H=16, N=1900, d=64, d_u=64, seed=3400 + int(scale))
    x = make_inputs(wl, u_scale=scale)
    o = run_causal(x, "bf16", rope=True)
    pairs = [(0, 1), (1, 12)]
    xs = slice_heads(x, pairs)
    ref = R.causal_forward(**xs, rope=True)
    got = np.stack([to_f64(o[b, h]) for b, h in pairs])[None]
    assert np.all(np.isfinite(got))
    err = rel_l2(got, ref)
    print(f"large logits x{scale} rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_causal_long_sequence_tail_precision():
    """Two heads at N = 16384 (128 scan segments of 2 chunks, so a long combine chain). Late in the
    sequence the outputs are small and the carried states nearly cancel against their H terms; the
    centred state basis keeps the error there at the level of the bf16 operand rounding. The bar
    for t > 1024 (6e-3, measured 3.9e-3) is tighter than the 2e-2 contract on purpose: a basis
    change that lets the states cancel before rounding doubles this error while staying under 2e-2."""
    wl = CONFIGS[4].with_(B=1, H=2, seed=3500)
    x = make_inputs(wl)
    o = run_causal(x, "bf16", rope=True)
    got = to_f64(o)
    ref = R.causal_forward(**x, rope=True)
    err = rel_l2(got, ref)
    tail = rel_l2(got[:, :, 1024:], ref[:, :, 1024:])
    print(f"long sequence rel_l2={err:.3e} tail={tail:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert tail <= 6e-3


def test_causal_one_head_very_long():
    """One head at N = 65536: 1024 chunks cut into 256 scan segments of 4 (a 255-step combine chain,
    loaded 8 segments at a time), and the precision of the carried states far past the lengths of
    the other tests."""
    wl = CONFIGS[4].with_(B=1, H=1, N=65536, seed=3600)
    x = make_inputs(wl)
    o = run_causal(x, "bf16", rope=True)
    got = to_f64(o)
    ref = R.causal_forward(**x, rope=True)
    err = rel_l2(got, ref)
    tail = rel_l2(got[:, :, 32768:], ref[:, :, 32768:])
    print(f"one head N=65536 rel_l2={err:.3e} tail(t>32768)={tail:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert tail <= TOL["bf16"]


def test_causal_workspace_reuse():
    wl = CONFIGS[4].with_(B=1, H=3, N=700, seed=3200)
    x = make_inputs(wl)
    t = to_device(x, "bf16")
    n = Z.zeros_fwd_causal_workspace_bytes(1, 3, 700, 128, 128, torch.bfloat16)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    args = [t[k] for k in ("q", "k", "v", "u", "mu", "tau", "g1", "gh")]
    o1 = Z.zeros_fwd_causal(*args, rope=True, workspace=ws)
    o2 = Z.zeros_fwd_causal(*args, rope=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert rel_l2(to_f64(o1), R.causal_forward(**x, rope=True)) <= TOL["bf16"]


def test_causal_f32_workspace_reuse():
    """The float32 path's workspace (logits, u sums, aggregates): a caller-owned buffer reused by two
    calls of different lengths gives the same outputs as calls that allocate their own."""
    ws = None
    for N in (700, 300):
        wl = CONFIGS[2].with_(B=2, H=3, N=N, seed=3250 + N)
        x = make_inputs(wl)
        t = to_device(x, "f32")
        if ws is None:
            n = Z.zeros_fwd_causal_workspace_bytes(2, 3, 700, 64, 64, torch.float32)
            assert n > 0
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        args = [t[k] for k in ("q", "k", "v", "u", "mu", "tau", "g1", "gh")]
        o1 = Z.zeros_fwd_causal(*args, workspace=ws)
        o2 = Z.zeros_fwd_causal(*args)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert rel_l2(to_f64(o1), R.causal_forward(**x)) <= TOL["f32"]


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("N", [1, 2, 47, 197])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rope", [False, True])
def test_encoder_shapes(d, N, dtype, rope):
    wl = CONFIGS[3].with_(B=2, H=2, N=N, d=d, d_u=d, dtype=dtype, seed=2000 + d + N)
    x = make_inputs(wl)
    o = to_f64(run_encoder(x, dtype, rope=rope))
    ref = R.encoder_forward(**x, rope=rope)
    if N == 1:
        assert np.max(np.abs(o)) <= ZERO_ABS    # one token: its weight is zero
    else:
        assert rel_l2(o, ref) <= TOL[dtype]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [64, 65, 128, 129, 255, 300, 700])
@pytest.mark.parametrize("rope", [False, True])
def test_encoder_mfma_chunks(d, N, rope):
    """bfloat16 encoder on the matrix cores: several 64-token state chunks and 16-token output
    blocks, ragged tails, both head dims; at d = 64 and N <= 256 the per-head variant, whose state
    pass stages 128 tokens per round (128 / 129: one or two rounds)."""
    wl = CONFIGS[3].with_(B=1, H=2, N=N, d=d, d_u=d, dtype="bf16", seed=3000 + d + N)
    x = make_inputs(wl)
    o = to_f64(run_encoder(x, "bf16", rope=rope))
    ref = R.encoder_forward(**x, rope=rope)
    err = rel_l2(o, ref)
    print(f"encoder mfma d={d} N={N} rope={rope} rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("d,N", [(64, 256), (64, 257), (128, 767), (128, 768), (64, 9000)])
def test_encoder_length_boundaries(d, N):
    """Sequence lengths at the edges of the encoder's variants: 256 / 257 tokens (per-head variant
    and the tile variant), 767 (the longest in one launch, logits in LDS), 768 and 9000 (the
    token-parallel pipeline with its scratch)."""
    wl = CONFIGS[3].with_(B=1, H=2, N=N, d=d, d_u=d, dtype="bf16", seed=3100 + d + N)
    x = make_inputs(wl)
    o = to_f64(run_encoder(x, "bf16", rope=True))
    ref = R.encoder_forward(**x, rope=True)
    err = rel_l2(o, ref)
    print(f"encoder d={d} N={N} rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("B,H,N,d,rope,gate0", [
    (1, 2, 4097, 64, False, False),     # last 256-token block holds one token
    (1, 2, 5000, 128, True, True),      # d = 128 with the zero-order gate (three states)
    (8, 8, 4500, 64, False, True),      # 64 heads: 512-token state blocks, the last one ragged
    (4, 8, 8192, 64, True, False),      # 32 heads: 512-token state blocks, 16 per head
    (2, 3, 6001, 128, False, False),    # d = 128, ragged tail inside an output block
    (96, 4, 300, 64, True, False),      # short sequences in a large batch: two 256-token blocks
    (1, 2, 768, 128, False, True),      # the shortest sequence that takes the pipeline on its own
])
def test_encoder_long_blocks(B, H, N, d, rope, gate0):
    """bfloat16 encoder on the token-parallel pipeline (u sums, logits per state block, partial
    states, their reduction, outputs): one and several 256-token spans per state block, ragged state
    and output blocks, RoPE and the zero-order gate."""
    wl = CONFIGS[3].with_(B=B, H=H, N=N, d=d, d_u=d, dtype="bf16", seed=3200 + B * H + N + d)
    x = make_inputs(wl, gate0=gate0)
    t = to_device(x, "bf16")
    o = Z.zeros_fwd_encoder(t["q"], t["k"], t["v"], t["u"], t["mu"], t["tau"], t["g1"], t["gh"],
                            g0=t["g0"] if gate0 else None, rope=rope)
    torch.cuda.synchronize()
    err = rel_l2(to_f64(o), R.encoder_forward(**x, rope=rope))
    print(f"encoder long B={B} H={H} N={N} d={d} rope={rope} gate0={gate0} rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_encoder_long_large_logits():
    """u scaled by 60 at N = 6000: the logits span about 300 (beyond the float32 exponent range of
    e^{+-88}), so the state blocks' (max, sum e^{s - max}) must be merged by rescaling to the
    global maximum, with the far-below blocks underflowing to zero weight."""
    wl = CONFIGS[3].with_(B=1, H=2, N=6000, d=64, d_u=64, dtype="bf16", seed=3998)
    x = make_inputs(wl, u_scale=60.0)
    o = to_f64(run_encoder(x, "bf16"))
    assert np.all(np.isfinite(o))
    assert rel_l2(o, R.encoder_forward(**x)) <= TOL["bf16"]


@pytest.mark.parametrize("N", [200, 300])
def test_encoder_mfma_large_logits(N):
    """u scaled by 30: logits spread over a wide range, the global maximum keeps e^{s-m} in range
    (N = 200: the per-head variant, N = 300: the tile variant)."""
    wl = CONFIGS[3].with_(B=1, H=2, N=N, d=64, d_u=64, dtype="bf16", seed=3999)
    x = make_inputs(wl, u_scale=30.0)
    o = to_f64(run_encoder(x, "bf16"))
    ref = R.encoder_forward(**x)
    assert rel_l2(o, ref) <= TOL["bf16"]


@pytest.mark.parametrize("scale", [10.0, 30.0])
def test_logit_stress_running_max(scale):
    """float32 inputs with u scaled by 10 and 30: the running maximum must keep e^{s} finite, and
    the 1e-4 contract still holds. At u x 30 the logits reach |s| of about 3.7e3, so float32
    rounding puts absolute errors of up to |s| 2^-24 = 2.2e-4 on them; but those extreme logits
    are the very negative ones at the start of the sequence, whose weights e^{s - m} vanish. Near
    the running maximum |s| <= 214, which bounds the relative error of e^{s - m} by 1.3e-5."""
    wl = CONFIGS[2].with_(B=1, H=4, N=300, seed=77)
    x = make_inputs(wl, u_scale=scale)
    o = to_f64(run_causal(x, "f32"))
    assert np.all(np.isfinite(o))
    err = rel_l2(o, R.causal_forward(**x))
    print(f"logit stress u x {scale}: rel_l2={err:.3e}", flush=True)
    assert err <= TOL["f32"]


def test_first_row_zero_and_constant_logits():
    wl = CONFIGS[2].with_(B=1, H=2, N=70, seed=78)
    x = make_inputs(wl)
    o = to_f64(run_causal(x, "f32"))
    assert np.max(np.abs(o[..., 0, :])) <= ZERO_ABS
    x["u"] = np.zeros_like(x["u"])
    assert np.max(np.abs(to_f64(run_causal(x, "f32")))) <= ZERO_ABS


def test_deterministic_and_causal():
    wl = CONFIGS[2].with_(B=2, H=2, N=200, seed=79)
    x = make_inputs(wl)
    o1 = run_causal(x, "f32").cpu()
    o2 = run_causal(x, "f32").cpu()
    assert torch.equal(o1, o2)
    y = {k: np.array(v, copy=True) for k, v in x.items()}
    rng = np.random.default_rng(5)
    for key in ("q", "k", "v", "u"):
        y[key][..., 150:, :] = rng.standard_normal(y[key][..., 150:, :].shape).astype(np.float32)
    o3 = run_causal(y, "f32").cpu()
    assert torch.equal(o1[..., :150, :], o3[..., :150, :])
    assert not torch.equal(o1[..., 150:, :], o3[..., 150:, :])


@pytest.mark.parametrize("cut", [640, 768])
def test_mfma_deterministic_and_causal(cut):
    """bfloat16 d 128 RoPE on the matrix-core path, 32 heads x 1500 tokens: 24 chunks in 8 scan
    segments of 3 (pass 1, combine, main). Two calls give identical bits; changing q, k, v, u and the
    gates of every token from a 64-token chunk boundary on leaves every earlier output bit for bit
    unchanged: 640 starts the second chunk of a segment (the chunk scan's reference maximum and the
    segment's pass-1 sums see the change only from there), 768 starts a segment and a 256-token
    logit segment."""
    wl = CONFIGS[4].with_(B=2, H=16, N=1500, seed=3800)
    x = make_inputs(wl)
    o1 = run_causal(x, "bf16", rope=True).cpu()
    o2 = run_causal(x, "bf16", rope=True).cpu()
    assert torch.equal(o1, o2)
    y = {k: np.array(v, copy=True) for k, v in x.items()}
    rng = np.random.default_rng(cut)
    for key in ("q", "k", "v", "u"):
        y[key][..., cut:, :] = rng.standard_normal(y[key][..., cut:, :].shape).astype(np.float32)
    for key in ("g1", "gh"):
        y[key][..., cut:] = rng.standard_normal(y[key][..., cut:].shape).astype(np.float32)
    o3 = run_causal(y, "bf16", rope=True).cpu()
    assert torch.equal(o1[..., :cut, :], o3[..., :cut, :])
    assert not torch.equal(o1[..., cut:, :], o3[..., cut:, :])


def test_side_stream_call():
    """A call launched on a side stream: the output and workspace the binding allocates belong to
    that stream, so allocations on the default stream while its kernels run cannot take their
    memory. Parity against the oracle after the side stream finishes."""
    wl = CONFIGS[4].with_(B=1, H=4, N=2000, seed=3900)
    x = make_inputs(wl)
    t = to_device(x, "bf16")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        o = Z.zeros_fwd_causal(t["q"], t["k"], t["v"], t["u"], t["mu"], t["tau"], t["g1"], t["gh"],
                               rope=True, stream=side)
        outs.append(o)
        # default-stream work that allocates and writes while the side stream's kernels may run
        junk = [torch.full((1 << 24,), 0x7F, dtype=torch.uint8, device="cuda") for _ in range(4)]
        del junk
    side.synchronize()
    ref = R.causal_forward(**x, rope=True)
    for o in outs:
        assert rel_l2(to_f64(o), ref) <= TOL["bf16"]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


# ------------------------------------------------------------------ state and decode

def _state_np(st):
    return {"F": to_f64(st.F), "G": to_f64(st.G), "H": to_f64(st.Hs), "Su": to_f64(st.Su),
            "m": to_f64(st.m), "E": to_f64(st.E), "P": to_f64(st.P),
            "t": st.t.cpu().numpy().astype(np.int64)}


@pytest.mark.parametrize("rope", [False, True])
def test_state_out_matches_oracle(rope):
    wl = CONFIGS[2].with_(B=2, H=3, N=77, d=32, d_u=32, seed=80)
    x = make_inputs(wl)
    st = Z.DecodeState(2, 3, 32, 32).reset()
    run_causal(x, "f32", rope=rope, state_out=st)
    _, ref = R.causal_forward(**x, rope=rope, return_state=True)
    got = _state_np(st)
    assert np.all(got["t"] == 77)
    for key in ("m", "E", "P", "Su", "F", "G", "H"):
        assert rel_l2(got[key], ref[key]) <= 1e-5, key


def test_state_out_empty_sequence():
    wl = CONFIGS[2].with_(B=1, H=2, N=0, d=16, d_u=16, seed=81)
    x = make_inputs(wl)
    st = Z.DecodeState(1, 2, 16, 16)
    st.buffer.fill_(0x7F)
    run_causal(x, "f32", state_out=st)
    assert torch.all(st.t == 0) and torch.all(torch.isneginf(st.m))
    for key in ("F", "G", "Hs", "Su", "E", "P"):
        assert torch.all(getattr(st, key) == 0), key


@pytest.mark.parametrize("dtype,rope", [("f32", False), ("f32", True), ("bf16", True)])
def test_decode_continues_forward(dtype, rope):
    wl = CONFIGS[2].with_(B=3, H=2, N=65, d=64, d_u=64, dtype=dtype, seed=82)
    x = make_inputs(wl)
    cut = 64
    head = {k: (v[..., :cut, :] if v.ndim == 4 else v[..., :cut] if v.ndim == 3 else v) for k, v in x.items()}
    st = Z.DecodeState(3, 2, 64, 64).reset()
    run_causal(head, dtype, rope=rope, state_out=st)
    t = to_device(x, dtype)
    o_step = Z.zeros_decode_step(t["q"][:, :, cut].contiguous(), t["k"][:, :, cut].contiguous(),
                                 t["v"][:, :, cut].contiguous(), t["u"][:, :, cut].contiguous(),
                                 t["mu"], t["tau"], t["g1"][:, :, cut].contiguous(),
                                 t["gh"][:, :, cut].contiguous(), st, rope=rope)
    torch.cuda.synchronize()
    ref = R.causal_forward(**x, rope=rope)[..., cut, :]
    assert rel_l2(to_f64(o_step), ref) <= TOL[dtype]
    assert torch.all(st.t == cut + 1)


def test_decode_from_empty_state_runs_the_recurrence():
    wl = CONFIGS[2].with_(B=2, H=2, N=20, d=16, d_u=16, seed=83)
    x = make_inputs(wl)
    t = to_device(x, "f32")
    st = Z.DecodeState(2, 2, 16, 16).reset()
    outs = []
    for n in range(20):
        outs.append(Z.zeros_decode_step(*(t[k][:, :, n].contiguous() for k in ("q", "k", "v", "u")),
                                        t["mu"], t["tau"], t["g1"][:, :, n].contiguous(),
                                        t["gh"][:, :, n].contiguous(), st))
    o = to_f64(torch.stack(outs, dim=2))
    assert rel_l2(o, R.causal_forward(**x)) <= TOL["f32"]


def test_config5_decode_full_size():
    """256 sequences x 32 heads, prefilled to t = 8192 with the causal forward, then one step.

    Parity: (a) the step from the GPU's own state, against the oracle step applied to that same
    state in float64, over every head; (b) the prefilled state of sampled (sequence, head) pairs
    against the oracle recurrence over their 8192 prefix tokens.
    """
    wl = CONFIGS[5]
    S, H, d = wl.B, wl.H, wl.d
    st = Z.DecodeState(S, H, d, d).reset()
    step = make_inputs(wl)
    t = to_device(step, wl.dtype)
    mu, tau = t["mu"], t["tau"]
    samples = [(0, 0), (200, 31)]
    sampled_prefix = {}
    batch = 16
    for s0 in range(0, S, batch):
        pre = decode_prefill_batch(wl, s0, s0 + batch)
        Z.zeros_fwd_causal(pre["q"], pre["k"], pre["v"], pre["u"], mu, tau, pre["g1"], pre["gh"],
                           state_out=st.sequences(s0, s0 + batch))
        for (s, h) in samples:
            if s0 <= s < s0 + batch:
                sampled_prefix[(s, h)] = {k: to_f64(val[s - s0, h]) for k, val in pre.items()}
        del pre
    torch.cuda.synchronize()
    assert torch.all(st.t == wl.prefill)
    # (b) sampled prefill states
    for (s, h), px in sampled_prefix.items():
        _, ref = R.causal_forward(px["q"], px["k"], px["v"], px["u"], step["mu"][h], step["tau"][h],
                                  px["g1"], px["gh"], return_state=True)
        for key, gk in (("F", st.F), ("G", st.G), ("H", st.Hs)):
            e = rel_l2(to_f64(gk[s, h]), ref[key])
            print(f"config5 prefill state ({s},{h}) {key}={e:.2e}", flush=True)
            assert e <= STATE_TOL_BF16, (s, h, key)
        assert abs(float(st.m[s, h]) - ref["m"]) <= SCALAR_STATE_TOL * max(1.0, abs(ref["m"]))
        assert rel_l2(to_f64(st.Su[s, h]), ref["Su"]) <= SCALAR_STATE_TOL
    # (a) one step from the identical state
    before = {k: getattr(st, a).cpu() for k, a in (("F", "F"), ("G", "G"), ("H", "Hs"), ("Su", "Su"),
                                                 ("m", "m"), ("E", "E"), ("P", "P"), ("t", "t"))}
    sq = {k: t[k][:, :, 0].contiguous() for k in ("q", "k", "v", "u", "g1", "gh")}
    o = Z.zeros_decode_step(sq["q"], sq["k"], sq["v"], sq["u"], mu, tau, sq["g1"], sq["gh"], st)
    torch.cuda.synchronize()
    o = to_f64(o)
    ref_o = np.empty_like(o)
    for s0 in range(0, S, 32):
        sl = slice(s0, s0 + 32)
        state = {k: v[sl].numpy().astype(np.float64 if k != "t" else np.int64) for k, v in before.items()}
        ref_o[sl], _ = R.decode_step(state, *(step[k][sl, :, 0] for k in ("q", "k", "v", "u")),
                                     step["mu"], step["tau"], step["g1"][sl, :, 0], step["gh"][sl, :, 0])
    err = rel_l2(o, ref_o)
    print(f"config5 step rel_l2={err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    assert torch.all(st.t == wl.prefill + 1)
