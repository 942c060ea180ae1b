"""ZeroS-SM on the GPU (zeros_sm_fwd_causal through the C ABI) against the float64 oracle.

The oracle is ``sm_causal_forward`` (pinned in tests/test_oracle_sm.py). Bars: bfloat16 inputs with
float32 accumulation, relative L2 of the whole output <= 2e-2 (the bfloat16 contract of every call);
the kernel also rounds the softmax weights and the logits to bfloat16 as matrix-core operands, like
any flash-style attention. The saturated-gate case is also checked against plain PyTorch float32
softmax attention of the same inputs.
"""
import numpy as np
import pytest
import torch

import zero_sum_attention_amd as Z
from oracle import zeros_ref as R

from .gpu_helpers import rel_l2, row_rel_p99, to_f64

pytestmark = pytest.mark.gpu
BAR = 2e-2


def _inputs(B, H, N, d, seed, g0=False, q_scale=1.0):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    x = {"q": bf(q_scale * rng.standard_normal((B, H, N, d))), "k": bf(rng.standard_normal((B, H, N, d))),
         "v": bf(rng.standard_normal((B, H, N, d))), "g1": bf(rng.standard_normal((B, H, N))),
         "gh": bf(rng.standard_normal((B, H, N)))}
    if g0:
        x["g0"] = bf(rng.standard_normal((B, H, N)))
    return x


def _run(x, rope=False):
    t = {k: v.cuda() for k, v in x.items()}
    o = Z.zeros_sm_fwd_causal(t["q"], t["k"], t["v"], t["g1"], t["gh"], g0=t.get("g0"), rope=rope)
    torch.cuda.synchronize()
    return o


def _oracle(x, rope=False, rows=None):
    f = {k: v.float().numpy().astype(np.float64) for k, v in x.items()}
    return R.sm_causal_forward(f["q"], f["k"], f["v"], f["g1"], f["gh"], rope=rope, g0=f.get("g0"), rows=rows)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 200])
@pytest.mark.parametrize("rope", [False, True])
def test_sm_shapes(d, N, rope):
    x = _inputs(2, 3, N, d, seed=100 + N + d)
    o = to_f64(_run(x, rope))
    ref = _oracle(x, rope)
    if N == 1:
        # one key: every part of the weight vanishes, so o_1 = 0 exactly
        assert np.max(np.abs(o)) <= 1e-6
        return
    err = rel_l2(o, ref)
    print(f"sm d={d} N={N} rope={rope} rel_l2={err:.3e} row_p99={row_rel_p99(o, ref, 1e-3):.3e}", flush=True)
    assert err <= BAR


@pytest.mark.parametrize("rope", [False, True])
def test_sm_zero_order_gate(rope):
    x = _inputs(1, 2, 333, 128, seed=7, g0=True)
    o = to_f64(_run(x, rope))
    err = rel_l2(o, _oracle(x, rope))
    print(f"sm g0 rope={rope} rel_l2={err:.3e}", flush=True)
    assert err <= BAR
    # first token: o_1 = sigma0_1 v_1 (one key; every other term of its weight is zero)
    s0 = torch.sigmoid(x["g0"][..., 0].float())
    np.testing.assert_allclose(o[..., 0, :], (s0[..., None] * x["v"][..., 0, :].float()).double().numpy(),
                               rtol=1e-2, atol=1e-2)


def test_sm_saturated_gates_match_torch_softmax_attention():
    """sigma1 = sigmah = sigma0 = 1 turns ZeroS-SM into standard causal softmax attention."""
    x = _inputs(2, 2, 150, 64, seed=9)
    big = torch.full(x["g1"].shape, 30.0).to(torch.bfloat16)
    x.update(g1=big, gh=big, g0=big)
    o = _run(x).float().cpu()
    q, k, v = (x[key].float() for key in ("q", "k", "v"))
    L = q @ k.transpose(-1, -2).contiguous() / 8.0
    L = L.masked_fill(~torch.tril(torch.ones(150, 150, dtype=torch.bool)), float("-inf"))
    ref = torch.softmax(L, dim=-1) @ v
    err = rel_l2(o.double().numpy(), ref.double().numpy())
    print(f"sm softmax limit rel_l2={err:.3e}", flush=True)
    assert err <= BAR


def test_sm_large_logits():
    """q scaled by 8: peaked softmax rows (the running maximum of the online softmax at work)."""
    x = _inputs(1, 2, 300, 128, seed=11, q_scale=8.0)
    o = to_f64(_run(x))
    err = rel_l2(o, _oracle(x))
    print(f"sm large logits rel_l2={err:.3e}", flush=True)
    assert err <= BAR


def test_sm_causal_and_deterministic():
    x = _inputs(1, 2, 320, 128, seed=13)
    o1 = _run(x, rope=True).cpu()
    o2 = _run(x, rope=True).cpu()
    assert torch.equal(o1, o2)
    y = {k: v.clone() for k, v in x.items()}
    for key in ("q", "k", "v"):
        y[key][..., 200:, :] = torch.randn(y[key][..., 200:, :].shape).to(torch.bfloat16)
    for key in ("g1", "gh"):
        y[key][..., 200:] = 0.5
    o3 = _run(y, rope=True).cpu()
    assert torch.equal(o1[..., :200, :], o3[..., :200, :])
    assert not torch.equal(o1[..., 200:, :], o3[..., 200:, :])


def test_sm_full_size_sampled_rows():
    """The long causal shape, B=2 H=16 N=16384 d=128 with RoPE: rows sampled across the sequence
    and the heads, each against the oracle row (O(t d) each); the whole output is finite."""
    B, H, N, d = 2, 16, 16384, 128
    gen = torch.Generator().manual_seed(17)
    x = {key: torch.randn((B, H, N, d), generator=gen).to(torch.bfloat16) for key in ("q", "k", "v")}
    x.update({key: torch.randn((B, H, N), generator=gen).to(torch.bfloat16) for key in ("g1", "gh")})
    o = _run(x, rope=True)
    assert torch.isfinite(o.float()).all()
    rows = [1, 2, 64, 65, 1000, 4097, 12345, 16384]
    for b, h in ((0, 0), (1, 15), (0, 7)):
        xs = {key: val[b, h] for key, val in x.items()}
        ref = _oracle(xs, rope=True, rows=rows)
        got = to_f64(o[b, h, [r - 1 for r in rows]])
        err = rel_l2(got, ref)
        print(f"sm full-size ({b},{h}) sampled rows rel_l2={err:.3e}", flush=True)
        assert err <= BAR


def test_sm_side_stream_and_workspace():
    x = _inputs(1, 2, 130, 64, seed=19)
    t = {k: v.cuda() for k, v in x.items()}
    n = Z.zeros_sm_fwd_causal_workspace_bytes(1, 2, 130, 64, torch.bfloat16, rope=True)
    assert n == 2 * 1 * 2 * 130 * 64 * 2
    assert Z.zeros_sm_fwd_causal_workspace_bytes(1, 2, 130, 64, torch.bfloat16, rope=False) == 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o = Z.zeros_sm_fwd_causal(t["q"], t["k"], t["v"], t["g1"], t["gh"], rope=True, workspace=ws, stream=s)
    s.synchronize()
    assert rel_l2(to_f64(o), _oracle(x, rope=True)) <= BAR
