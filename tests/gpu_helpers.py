"""Shared helpers of the GPU tests: device transfer of seeded inputs and error metrics."""
import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
# Tolerances on the relative L2 error of the whole output tensor:
#   float32 inputs: 1e-4; bfloat16 inputs with float32 accumulation: 2e-2.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_device(x: dict, dtype: str, device="cuda"):
    """Seeded numpy inputs (already rounded to dtype) -> torch tensors on the GPU."""
    out = {}
    for key, val in x.items():
        t = torch.from_numpy(np.ascontiguousarray(val))
        if key in ("mu", "tau"):
            out[key] = t.to(device=device, dtype=torch.float32)
        else:
            out[key] = t.to(device=device, dtype=TORCH_DT[dtype])
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def tail_rel_l2(a, b, start: int) -> float:
    return rel_l2(np.asarray(a)[..., start:, :], np.asarray(b)[..., start:, :])


def slice_heads(x: dict, pairs):
    """Inputs of the (b, h) pairs only, as [1, len(pairs), ...] arrays (mu, tau per pair)."""
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    out = {}
    for key, val in x.items():
        if key == "mu":
            out[key] = val[hs]
        elif key == "tau":
            out[key] = val[hs]
        else:
            out[key] = val[bs, hs][None]
    return out
