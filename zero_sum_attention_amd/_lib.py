"""ctypes binding of libzeros (argument marshalling only; every step runs in the HIP kernels).

Tensors are torch tensors on the GPU: torch supplies device memory and the current stream. The
functions check shapes, dtypes, devices and contiguity (the C library cannot see tensor sizes),
then pass raw pointers. A missing or unloadable libzeros.so raises immediately: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzeros.so")

ZEROS_OK, ZEROS_ERR_NULL, ZEROS_ERR_SHAPE, ZEROS_ERR_DTYPE = 0, 1, 2, 3
ZEROS_ERR_UNSUPPORTED, ZEROS_ERR_HIP, ZEROS_ERR_ALIAS = 4, 5, 6
ZEROS_F32, ZEROS_BF16 = 0, 1
_DT = {torch.float32: ZEROS_F32, torch.bfloat16: ZEROS_BF16}


class ZerosError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class zeros_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("d_u", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope", ctypes.c_int32), ("rope_base", ctypes.c_float)]


class zeros_state(ctypes.Structure):
    _fields_ = [("F", ctypes.c_void_p), ("G", ctypes.c_void_p), ("Hs", ctypes.c_void_p),
                ("Su", ctypes.c_void_p), ("m", ctypes.c_void_p), ("E", ctypes.c_void_p),
                ("P", ctypes.c_void_p), ("t", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libzeros.so (once) and declare its exported signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m zero_sum_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    # shape, q, k, v, u, mu, tau, g1, gh, g0, o
    fwd = [ctypes.POINTER(zeros_shape), vp, vp, vp, vp, f32p, f32p, vp, vp, vp, vp]
    lib.zeros_fwd_causal.argtypes = fwd + [ctypes.POINTER(zeros_state), ctypes.POINTER(zeros_state), vp,
                                           ctypes.c_size_t, vp]
    lib.zeros_fwd_causal.restype = i32
    lib.zeros_fwd_causal_noalloc.argtypes = fwd + [ctypes.POINTER(zeros_state), ctypes.POINTER(zeros_state), vp]
    lib.zeros_fwd_causal_noalloc.restype = i32
    lib.zeros_fwd_causal_workspace_bytes.argtypes = [ctypes.POINTER(zeros_shape)]
    lib.zeros_fwd_causal_workspace_bytes.restype = ctypes.c_size_t
    lib.zeros_fwd_encoder.argtypes = fwd + [vp, ctypes.c_size_t, vp]
    lib.zeros_fwd_encoder.restype = i32
    lib.zeros_fwd_encoder_workspace_bytes.argtypes = [ctypes.POINTER(zeros_shape)]
    lib.zeros_fwd_encoder_workspace_bytes.restype = ctypes.c_size_t
    lib.zeros_decode_step.argtypes = fwd + [ctypes.POINTER(zeros_state), vp]
    lib.zeros_decode_step.restype = i32
    lib.zeros_bwd_causal.argtypes = fwd[:10] + [vp] * 5 + [f32p, f32p] + [vp] * 3 + [vp, ctypes.c_size_t, vp]
    lib.zeros_bwd_causal.restype = i32
    lib.zeros_bwd_causal_workspace_bytes.argtypes = [ctypes.POINTER(zeros_shape)]
    lib.zeros_bwd_causal_workspace_bytes.restype = ctypes.c_size_t
    # shape, q, k, v, g1, gh, g0, o, workspace, workspace_bytes, stream
    lib.zeros_sm_fwd_causal.argtypes = [ctypes.POINTER(zeros_shape), vp, vp, vp, vp, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp]
    lib.zeros_sm_fwd_causal.restype = i32
    lib.zeros_sm_fwd_causal_workspace_bytes.argtypes = [ctypes.POINTER(zeros_shape)]
    lib.zeros_sm_fwd_causal_workspace_bytes.restype = ctypes.c_size_t
    lib.zeros_state_bytes.argtypes = [i32, i32, i32, i32]
    lib.zeros_state_bytes.restype = ctypes.c_size_t
    lib.zeros_state_from_buffer.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(zeros_state)]
    lib.zeros_state_from_buffer.restype = i32
    lib.zeros_status_str.argtypes = [i32]
    lib.zeros_status_str.restype = ctypes.c_char_p
    lib.zeros_last_error.argtypes = []
    lib.zeros_last_error.restype = ctypes.c_char_p
    lib.zeros_abi_version.argtypes = []
    lib.zeros_abi_version.restype = i32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != ZEROS_OK:
        lib = load_library()
        raise ZerosError(status, lib.zeros_last_error().decode() or lib.zeros_status_str(status).decode())


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> torch.cuda.Stream:
    """The stream the call's kernels are launched on (the current stream by default)."""
    return torch.cuda.current_stream(device) if stream is None else stream


def _alloc_on(stream: torch.cuda.Stream, fn):
    """Allocate through torch's caching allocator as the launch stream's memory: a block freed
    after the call is reused only by later work on that same stream, so it cannot be handed to
    another stream while the call's kernels still use it."""
    with torch.cuda.stream(stream):
        return fn()


def _workspace(nbytes: int, workspace, device, stream):
    if workspace is None and nbytes > 0:
        workspace = _alloc_on(stream, lambda: torch.empty(nbytes, dtype=torch.uint8, device=device))
    if workspace is not None:
        _need(workspace.dtype == torch.uint8 and workspace.device == device and workspace.is_contiguous(),
              "workspace must be a contiguous uint8 tensor on q's device")
    return workspace


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_tensors(q, k, v, u, mu, tau, g1, gh, n_tok_dims: int, g0=None):
    """Validate [B, H, N, d] (n_tok_dims = 1) or [S, H, d] (n_tok_dims = 0) tensors."""
    _need(q.dtype in _DT, f"q dtype {q.dtype} is not float32 or bfloat16")
    dev = q.device
    _need(dev.type == "cuda", "tensors must be on a GPU")
    gates = (("g1", g1), ("gh", gh)) + ((("g0", g0),) if g0 is not None else ())
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u)) + gates:
        _need(t.dtype == q.dtype, f"{name} dtype {t.dtype} differs from q ({q.dtype})")
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u), ("mu", mu), ("tau", tau)) + gates:
        _need(t.device == dev, f"{name} is on {t.device}, q on {dev}")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(mu.dtype == torch.float32 and tau.dtype == torch.float32, "mu and tau must be float32")
    nd = 3 + n_tok_dims
    _need(q.dim() == nd, f"q must have {nd} dims")
    _need(k.shape == q.shape and v.shape == q.shape, "q, k, v shapes differ")
    _need(u.shape[:-1] == q.shape[:-1], "u leading dims differ from q")
    _need(all(t.shape == q.shape[:-1] for _, t in gates), "gate shapes must be q.shape[:-1]")
    H, du = q.shape[1], u.shape[-1]
    _need(mu.shape == (H, du), f"mu must be [H, d_u] = [{H}, {du}]")
    _need(tau.shape == (H,), f"tau must be [H] = [{H}]")


def _shape(q, u, n_tok: int, rope: bool, rope_base: float) -> zeros_shape:
    return zeros_shape(q.shape[0], q.shape[1], n_tok, q.shape[-1], u.shape[-1], _DT[q.dtype],
                       1 if rope else 0, float(rope_base))


class DecodeState:
    """Device buffers of a recurrent state for S sequences x H heads (layout of zeros_state)."""

    def __init__(self, S: int, H: int, d: int, d_u: int, device="cuda"):
        lib = load_library()
        nbytes = lib.zeros_state_bytes(S, H, d, d_u)
        _need(nbytes > 0, "invalid state sizes")
        self.S, self.H, self.d, self.d_u = S, H, d, d_u
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = zeros_state()
        _check(lib.zeros_state_from_buffer(ctypes.c_void_p(self.buffer.data_ptr()), S, H, d, d_u,
                                           ctypes.byref(self.c)))
        base = self.buffer.data_ptr()

        def view(addr, n, dtype, shape):
            off = addr - base
            return self.buffer[off:off + n * 4].view(dtype).view(*shape)

        n = S * H
        self.F = view(self.c.F, n * d * d, torch.float32, (S, H, d, d))
        self.G = view(self.c.G, n * d * d, torch.float32, (S, H, d, d))
        self.Hs = view(self.c.Hs, n * d * d, torch.float32, (S, H, d, d))
        self.Su = view(self.c.Su, n * d_u, torch.float32, (S, H, d_u))
        self.m = view(self.c.m, n, torch.float32, (S, H))
        self.E = view(self.c.E, n, torch.float32, (S, H))
        self.P = view(self.c.P, n, torch.float32, (S, H))
        self.t = view(self.c.t, n, torch.int32, (S, H))

    def sequences(self, s0: int, s1: int) -> "DecodeState":
        """A view of sequences [s0, s1) sharing this state's memory."""
        _need(0 <= s0 < s1 <= self.S, "sequence range out of bounds")
        view = DecodeState.__new__(DecodeState)
        view.S, view.H, view.d, view.d_u = s1 - s0, self.H, self.d, self.d_u
        view.buffer = self.buffer
        n0 = s0 * self.H
        mat, vec = self.d * self.d * 4, self.d_u * 4
        view.c = zeros_state(self.c.F + n0 * mat, self.c.G + n0 * mat, self.c.Hs + n0 * mat,
                             self.c.Su + n0 * vec, self.c.m + n0 * 4, self.c.E + n0 * 4,
                             self.c.P + n0 * 4, self.c.t + n0 * 4)
        for name in ("F", "G", "Hs", "Su", "m", "E", "P", "t"):
            setattr(view, name, getattr(self, name)[s0:s1])
        return view

    def reset(self) -> "DecodeState":
        """Set every head to the empty state (t = 0, m = -inf, sums zero)."""
        self.buffer.zero_()
        self.m.fill_(float("-inf"))
        return self


def zeros_fwd_causal(q, k, v, u, mu, tau, g1, gh, *, g0: torch.Tensor | None = None, rope: bool = False,
                     rope_base: float = 10000.0, out: torch.Tensor | None = None,
                     state_in: DecodeState | None = None, state_out: DecodeState | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Causal forward over q, k, v [B, H, N, d], u [B, H, N, d_u], g1, gh [B, H, N].

    ``g0`` [B, H, N] (optional) enables the zero-order gate. ``state_in`` continues every
    (b, h) from a state (chunked prefill); ``state_out`` receives the final state and must be a
    different state object. ``workspace`` (optional uint8 tensor) is reused scratch; without it
    one is allocated per call when the path needs it (see zeros_fwd_causal_workspace_bytes).
    ``stream`` (a torch.cuda.Stream, default the current one) receives the kernels; the output
    and the workspace allocated here belong to it."""
    _check_tensors(q, k, v, u, mu, tau, g1, gh, 1, g0)
    s_ = _stream(q.device, stream)
    o = _alloc_on(s_, lambda: torch.empty_like(v)) if out is None else out
    _need(o.shape == v.shape and o.dtype == v.dtype and o.is_contiguous() and o.device == q.device,
          "out must match v")
    for name, st_ in (("state_in", state_in), ("state_out", state_out)):
        if st_ is not None:
            _need((st_.S, st_.H, st_.d, st_.d_u) == (q.shape[0], q.shape[1], q.shape[-1], u.shape[-1]),
                  f"{name} sizes differ")
    lib = load_library()
    shp = _shape(q, u, q.shape[2], rope, rope_base)
    st = ctypes.byref(state_out.c) if state_out is not None else None
    sti = ctypes.byref(state_in.c) if state_in is not None else None
    nws = lib.zeros_fwd_causal_workspace_bytes(ctypes.byref(shp))
    workspace = _workspace(nws, workspace, q.device, s_)
    _check(lib.zeros_fwd_causal(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(mu),
                                _ptr(tau), _ptr(g1), _ptr(gh), _ptr(g0), _ptr(o), sti, st,
                                _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                s_.cuda_stream))
    return o


def zeros_fwd_causal_noalloc(q, k, v, u, mu, tau, g1, gh, *, g0: torch.Tensor | None = None, rope: bool = False,
                             rope_base: float = 10000.0, out: torch.Tensor | None = None,
                             state_in: DecodeState | None = None, state_out: DecodeState | None = None,
                             stream=None) -> torch.Tensor:
    """zeros_fwd_causal through the entry point that allocates nothing (its scratch is a fixed
    per-GPU array of ZEROS_NOALLOC_SCRATCH_BYTES). Calls that overlap on one GPU race; ``out``
    lets the caller avoid torch's allocation of the output as well."""
    _check_tensors(q, k, v, u, mu, tau, g1, gh, 1, g0)
    s_ = _stream(q.device, stream)
    o = _alloc_on(s_, lambda: torch.empty_like(v)) if out is None else out
    _need(o.shape == v.shape and o.dtype == v.dtype and o.is_contiguous() and o.device == q.device,
          "out must match v")
    for name, st_ in (("state_in", state_in), ("state_out", state_out)):
        if st_ is not None:
            _need((st_.S, st_.H, st_.d, st_.d_u) == (q.shape[0], q.shape[1], q.shape[-1], u.shape[-1]),
                  f"{name} sizes differ")
    lib = load_library()
    shp = _shape(q, u, q.shape[2], rope, rope_base)
    _check(lib.zeros_fwd_causal_noalloc(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(mu),
                                        _ptr(tau), _ptr(g1), _ptr(gh), _ptr(g0), _ptr(o),
                                        ctypes.byref(state_in.c) if state_in is not None else None,
                                        ctypes.byref(state_out.c) if state_out is not None else None,
                                        s_.cuda_stream))
    return o


def zeros_fwd_causal_workspace_bytes(B: int, H: int, N: int, d: int, d_u: int, dtype, rope: bool = False) -> int:
    """Scratch bytes zeros_fwd_causal needs for these sizes (0 when the path needs none)."""
    lib = load_library()
    shp = zeros_shape(B, H, N, d, d_u, _DT[dtype], 1 if rope else 0, 10000.0)
    return int(lib.zeros_fwd_causal_workspace_bytes(ctypes.byref(shp)))


def zeros_fwd_encoder(q, k, v, u, mu, tau, g1, gh, *, g0: torch.Tensor | None = None, rope: bool = False,
                      rope_base: float = 10000.0, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Non-causal forward; same tensor layout (and optional ``g0``) as zeros_fwd_causal.
    ``workspace`` as for zeros_fwd_causal (only long bfloat16 sequences need one)."""
    _check_tensors(q, k, v, u, mu, tau, g1, gh, 1, g0)
    s_ = _stream(q.device, stream)
    o = _alloc_on(s_, lambda: torch.empty_like(v)) if out is None else out
    _need(o.shape == v.shape and o.dtype == v.dtype and o.is_contiguous() and o.device == q.device,
          "out must match v")
    lib = load_library()
    shp = _shape(q, u, q.shape[2], rope, rope_base)
    workspace = _workspace(lib.zeros_fwd_encoder_workspace_bytes(ctypes.byref(shp)), workspace, q.device, s_)
    _check(lib.zeros_fwd_encoder(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(mu),
                                 _ptr(tau), _ptr(g1), _ptr(gh), _ptr(g0), _ptr(o),
                                 _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                 s_.cuda_stream))
    return o


def zeros_fwd_encoder_workspace_bytes(B: int, H: int, N: int, d: int, d_u: int, dtype) -> int:
    """Scratch bytes zeros_fwd_encoder needs for these sizes (0 when it needs none)."""
    lib = load_library()
    shp = zeros_shape(B, H, N, d, d_u, _DT[dtype], 0, 10000.0)
    return int(lib.zeros_fwd_encoder_workspace_bytes(ctypes.byref(shp)))


def zeros_sm_fwd_causal(q, k, v, g1, gh, *, g0: torch.Tensor | None = None, rope: bool = False,
                        rope_base: float = 10000.0, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """ZeroS-SM, causal: the zero-sum reweighting of standard softmax attention. q, k, v [B, H, N, d]
    bfloat16 (d 64 or 128), g1, gh (and g0) [B, H, N] bfloat16. ``workspace`` (rotated q and k, with
    RoPE only) as for zeros_fwd_causal."""
    _need(q.dim() == 4 and k.shape == q.shape and v.shape == q.shape, "q, k, v must be [B, H, N, d]")
    _need(q.dtype in _DT, f"q dtype {q.dtype} is not float32 or bfloat16")
    _need(g1.shape == q.shape[:3] and gh.shape == q.shape[:3] and (g0 is None or g0.shape == q.shape[:3]),
          "g1, gh, g0 must be [B, H, N]")
    for t in (q, k, v, g1, gh) + (() if g0 is None else (g0,)):
        _need(t.is_contiguous() and t.device == q.device and t.dtype == q.dtype, "tensors must be contiguous, "
              "on one device and of one dtype")
    s_ = _stream(q.device, stream)
    o = _alloc_on(s_, lambda: torch.empty_like(v)) if out is None else out
    _need(o.shape == v.shape and o.dtype == v.dtype and o.is_contiguous() and o.device == q.device,
          "out must match v")
    lib = load_library()
    B, H, N, d = q.shape
    shp = zeros_shape(B, H, N, d, d, _DT[q.dtype], int(rope), float(rope_base))
    workspace = _workspace(lib.zeros_sm_fwd_causal_workspace_bytes(ctypes.byref(shp)), workspace, q.device, s_)
    _check(lib.zeros_sm_fwd_causal(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(g1), _ptr(gh), _ptr(g0),
                                   _ptr(o), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                   s_.cuda_stream))
    return o


def zeros_sm_fwd_causal_workspace_bytes(B: int, H: int, N: int, d: int, dtype, rope: bool = False) -> int:
    """Scratch bytes zeros_sm_fwd_causal needs for these sizes (0 without RoPE)."""
    lib = load_library()
    shp = zeros_shape(B, H, N, d, d, _DT[dtype], int(rope), 10000.0)
    return int(lib.zeros_sm_fwd_causal_workspace_bytes(ctypes.byref(shp)))


def zeros_decode_step(q, k, v, u, mu, tau, g1, gh, state: DecodeState, *, g0: torch.Tensor | None = None,
                      rope: bool = False, rope_base: float = 10000.0, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """One token per (sequence, head): q, k, v [S, H, d], u [S, H, d_u], g1, gh (and g0) [S, H]."""
    _check_tensors(q, k, v, u, mu, tau, g1, gh, 0, g0)
    _need((state.S, state.H, state.d, state.d_u) == (q.shape[0], q.shape[1], q.shape[-1], u.shape[-1]),
          "state sizes differ from the token tensors")
    s_ = _stream(q.device, stream)
    o = _alloc_on(s_, lambda: torch.empty_like(v)) if out is None else out
    _need(o.shape == v.shape and o.dtype == v.dtype and o.is_contiguous() and o.device == q.device,
          "out must match v")
    lib = load_library()
    shp = _shape(q, u, 1, rope, rope_base)
    _check(lib.zeros_decode_step(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(mu),
                                 _ptr(tau), _ptr(g1), _ptr(gh), _ptr(g0), _ptr(o), ctypes.byref(state.c),
                                 s_.cuda_stream))
    return o


def zeros_bwd_causal(q, k, v, u, mu, tau, g1, gh, dO, *, g0: torch.Tensor | None = None, rope: bool = False,
                     rope_base: float = 10000.0, workspace: torch.Tensor | None = None, stream=None) -> dict:
    """Gradients of sum(dO * zeros_fwd_causal(...)) for every input (the backward of the causal
    forward from the empty state). Returns a dict with q, k, v, u, g1, gh (and g0) in the input
    dtype and mu [H, d_u], tau [H] in float32, summed over the batch."""
    _check_tensors(q, k, v, u, mu, tau, g1, gh, 1, g0)
    _need(dO.shape == v.shape and dO.dtype == v.dtype and dO.is_contiguous() and dO.device == q.device,
          "dO must match v")
    s_ = _stream(q.device, stream)
    lib = load_library()
    shp = _shape(q, u, q.shape[2], rope, rope_base)

    def alloc():
        out = {"q": torch.empty_like(q), "k": torch.empty_like(k), "v": torch.empty_like(v),
               "u": torch.empty_like(u), "g1": torch.empty_like(g1), "gh": torch.empty_like(gh),
               "mu": torch.empty_like(mu), "tau": torch.empty_like(tau)}
        if g0 is not None:
            out["g0"] = torch.empty_like(g0)
        return out

    g = _alloc_on(s_, alloc)
    workspace = _workspace(lib.zeros_bwd_causal_workspace_bytes(ctypes.byref(shp)), workspace, q.device, s_)
    _check(lib.zeros_bwd_causal(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(mu), _ptr(tau),
                                _ptr(g1), _ptr(gh), _ptr(g0), _ptr(dO), _ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]),
                                _ptr(g["u"]), _ptr(g["mu"]), _ptr(g["tau"]), _ptr(g["g1"]), _ptr(g["gh"]),
                                _ptr(g.get("g0")), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                s_.cuda_stream))
    return g


def zeros_bwd_causal_workspace_bytes(B: int, H: int, N: int, d: int, d_u: int, dtype) -> int:
    """Scratch bytes zeros_bwd_causal needs for these sizes."""
    lib = load_library()
    shp = zeros_shape(B, H, N, d, d_u, _DT[dtype], 0, 10000.0)
    return int(lib.zeros_bwd_causal_workspace_bytes(ctypes.byref(shp)))
