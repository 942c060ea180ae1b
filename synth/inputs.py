"""Workload table and seeded input generator.

Every tensor is drawn with ``numpy.random.default_rng(seed)`` (PCG64) in float32, in the fixed
order q, k, v, u, mu, tau, g1, gh, and then rounded to the workload's storage dtype. The
rounded values are returned as float32 arrays; whoever consumes them (the float64 oracle or the
GPU library) sees exactly the same numbers.

Distributions: q, k, v, u ~ N(0, 1) iid; mu ~ N(0, 0.1^2) per head; tau is either 0 or
U(-1, 1) per head; the gate pre-activations g1, gh ~ N(0, 1) per token.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    d_u: int
    dtype: str          # "f32" or "bf16": storage type of q, k, v, u, g1, gh and o
    mode: str           # "causal", "encoder" or "decode"
    rope: bool = False
    rope_base: float = 10000.0
    tau_uniform: bool = False   # tau ~ U(-1, 1) per head when True, else tau = 0
    seed: int = 0
    prefill: int = 0    # decode only: tokens already folded into the state

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.B * self.N

    def summary(self) -> dict:
        out = {"workload": self.name, "mode": self.mode, "B": self.B, "H": self.H,
               "N": self.N, "d": self.d, "d_u": self.d_u, "dtype": self.dtype,
               "rope": self.rope, "seed": self.seed}
        if self.mode == "decode":
            out["prefill"] = self.prefill
        return out


CONFIGS = {
    1: Workload("tiny-causal-B1H1N64d16", 1, 1, 64, 16, 16, "f32", "causal", seed=1),
    2: Workload("lm-layer-causal-B8H8N512d64", 8, 8, 512, 64, 64, "f32", "causal",
                tau_uniform=True, seed=2),
    3: Workload("vit-tiny-encoder-B64H3N197d64", 64, 3, 197, 64, 64, "bf16", "encoder", seed=3),
    4: Workload("long-causal-rope-B2H16N16384d128", 2, 16, 16384, 128, 128, "bf16", "causal",
                rope=True, tau_uniform=True, seed=4),
    5: Workload("decode-S256H32d128-t8192", 256, 32, 1, 128, 128, "bf16", "decode",
                tau_uniform=True, seed=5, prefill=8192),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # finite inputs stay below 2^32 after the rounding add; NaN is passed through unchanged
    rounded = (bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    out = rounded.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, x, out)
    return out


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(wl: Workload, *, u_scale: float = 1.0, gate0: bool = False, grad_out: bool = False) -> dict:
    """Draw one batch of inputs for ``wl``.

    Shapes: q, k, v [B, H, N, d]; u [B, H, N, d_u]; mu [H, d_u]; tau [H]; g1, gh [B, H, N].
    For decode workloads N is 1 (one new token per sequence). ``u_scale`` multiplies u before
    rounding (logit stress cases). ``gate0`` adds zero-order gate pre-activations g0 ~ N(0, 1)
    [B, H, N], drawn after everything else so the other inputs do not change. ``grad_out`` adds
    an upstream gradient dO ~ N(0, 1) [B, H, N, d] (the backward pass's input), drawn last.
    """
    rng = np.random.default_rng(wl.seed)
    B, H, N, d, du = wl.B, wl.H, wl.N, wl.d, wl.d_u
    q = rng.standard_normal((B, H, N, d), dtype=np.float32)
    k = rng.standard_normal((B, H, N, d), dtype=np.float32)
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    u = rng.standard_normal((B, H, N, du), dtype=np.float32)
    mu = (0.1 * rng.standard_normal((H, du), dtype=np.float32)).astype(np.float32)
    if wl.tau_uniform:
        tau = rng.uniform(-1.0, 1.0, size=(H,)).astype(np.float32)
    else:
        tau = np.zeros((H,), dtype=np.float32)
    g1 = rng.standard_normal((B, H, N), dtype=np.float32)
    gh = rng.standard_normal((B, H, N), dtype=np.float32)
    if u_scale != 1.0:
        u = (u * np.float32(u_scale)).astype(np.float32)
    dt = wl.dtype
    out = {
        "q": round_to_dtype(q, dt), "k": round_to_dtype(k, dt), "v": round_to_dtype(v, dt),
        "u": round_to_dtype(u, dt), "mu": mu, "tau": tau,
        "g1": round_to_dtype(g1, dt), "gh": round_to_dtype(gh, dt),
    }
    if gate0:
        out["g0"] = round_to_dtype(rng.standard_normal((B, H, N), dtype=np.float32), dt)
    if grad_out:
        out["dO"] = round_to_dtype(rng.standard_normal((B, H, N, d), dtype=np.float32), dt)
    return out


def decode_prefill_batch(wl: Workload, s0: int, s1: int, device="cuda"):
    """Prefix tokens 1..wl.prefill of decode sequences [s0, s1), drawn on the GPU.

    The full prefix of a decode workload (256 x 32 x 8192 tokens x 4 tensors) is far too large to
    draw on the host, so it comes from torch's device generator seeded with (wl.seed, s0): the
    same batch always gets the same values on the same software stack. Returns torch tensors
    q, k, v, u [s1-s0, H, prefill, d] and g1, gh [s1-s0, H, prefill] in the workload dtype.
    """
    import torch

    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[wl.dtype]
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1_000_003 + s0)
    S, H, T = s1 - s0, wl.H, wl.prefill
    out = {}
    for key in ("q", "k", "v", "u"):
        feat = wl.d_u if key == "u" else wl.d
        out[key] = torch.randn((S, H, T, feat), generator=g, device=device, dtype=torch.float32).to(dt)
    for key in ("g1", "gh"):
        out[key] = torch.randn((S, H, T), generator=g, device=device, dtype=torch.float32).to(dt)
    return out
