"""The no-allocation causal entry point (zeros_fwd_causal_noalloc, through the C ABI) gives the
results of zeros_fwd_causal with a workspace, on two calls in a row on the same GPU (the second
smaller, so it reuses the fixed scratch the first one left behind), on both causal paths."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, make_inputs
from tests.gpu_helpers import TOL, rel_l2, to_device, to_f64

pytestmark = pytest.mark.gpu

import zero_sum_attention_amd as Z  # noqa: E402

KEYS = ("q", "k", "v", "u", "mu", "tau", "g1", "gh")


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,d,rope,sizes", [
    ("bf16", 128, True, [(2, 4, 1500), (1, 2, 300)]),      # matrix-core path, several scan segments
    ("bf16", 64, False, [(1, 3, 700), (1, 1, 65)]),
    ("f32", 64, True, [(2, 3, 900), (1, 2, 100)]),        # float32 path
])
def test_noalloc_matches_workspace_call(dtype, d, rope, sizes):
    for i, (B, H, N) in enumerate(sizes):
        wl = CONFIGS[2].with_(B=B, H=H, N=N, d=d, d_u=d, dtype=dtype, seed=7000 + 10 * i + d)
        x = make_inputs(wl)
        t = to_device(x, dtype)
        args = [t[k] for k in KEYS]
        ref = Z.zeros_fwd_causal(*args, rope=rope)
        st_a = Z.DecodeState(B, H, d, d).reset()
        st_b = Z.DecodeState(B, H, d, d).reset()
        Z.zeros_fwd_causal(*args, rope=rope, state_out=st_a)
        got = Z.zeros_fwd_causal_noalloc(*args, rope=rope, state_out=st_b)
        torch.cuda.synchronize()
        err = rel_l2(to_f64(got), to_f64(ref))
        print(f"noalloc {dtype} d={d} B{B} H{H} N{N}: rel_l2 vs workspace call {err:.2e}", flush=True)
        assert err <= TOL[dtype]
        assert torch.equal(got, ref)              # same kernels on the same inputs: same bits
        for name in ("F", "G", "Hs", "Su", "m", "E", "P", "t"):
            assert torch.equal(getattr(st_a, name), getattr(st_b, name)), name


def test_noalloc_continued_call():
    """state_in through the no-allocation entry point: a prefix, then the rest from its state."""
    wl = CONFIGS[4].with_(B=1, H=2, N=700, seed=7100)
    x = make_inputs(wl)
    t = to_device(x, "bf16")
    part = lambda a, b: [(t[k][:, :, a:b].contiguous() if k not in ("mu", "tau") else t[k]) for k in KEYS]  # noqa: E731
    s1, s2 = Z.DecodeState(1, 2, 128, 128).reset(), Z.DecodeState(1, 2, 128, 128).reset()
    Z.zeros_fwd_causal_noalloc(*part(0, 300), rope=True, state_out=s1)
    Z.zeros_fwd_causal(*part(0, 300), rope=True, state_out=s2)
    a = Z.zeros_fwd_causal_noalloc(*part(300, 700), rope=True, state_in=s1)
    b = Z.zeros_fwd_causal(*part(300, 700), rope=True, state_in=s2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_noalloc_rejects_oversize():
    """A call whose scratch would exceed the fixed array is refused before any launch (64 heads
    of 262144 tokens: 67 MB of float32 logits alone)."""
    B, H, N, d = 1, 64, 262144, 16
    need = Z.zeros_fwd_causal_workspace_bytes(B, H, N, d, d, torch.bfloat16, False)
    assert need > (64 << 20)
    q = torch.zeros(B, H, N, d, device="cuda", dtype=torch.bfloat16)
    gate = torch.zeros(B, H, N, device="cuda", dtype=torch.bfloat16)
    mu, tau = torch.zeros(H, d, device="cuda"), torch.zeros(H, device="cuda")
    with pytest.raises(Z.ZerosError, match="more than the fixed"):
        Z.zeros_fwd_causal_noalloc(q, q.clone(), q.clone(), q.clone(), mu, tau, gate, gate.clone())
