"""C-ABI tests that need no GPU: the library loads, exports every function the header declares,
and rejects bad arguments on the host before any HIP call.

Every call here that passes placeholder pointers is one that validation rejects (or a no-op such
as N = 0 without a state), so no kernel is ever launched with them.
"""
import ctypes
import os
import re

import pytest

from zero_sum_attention_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zeros.h")


@pytest.fixture(scope="module")
def lib():
    return L.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zeros_[a-z_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("zeros_fwd_causal", "zeros_fwd_encoder", "zeros_decode_step", "zeros_state_bytes",
              "zeros_fwd_causal_workspace_bytes", "zeros_fwd_encoder_workspace_bytes",
              "zeros_state_from_buffer", "zeros_status_str", "zeros_last_error", "zeros_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libzeros.so does not export {name}"


def test_abi_version(lib):
    text = open(HEADER).read()
    ver = int(re.search(r"#define ZEROS_ABI_VERSION (\d+)", text).group(1))
    assert lib.zeros_abi_version() == ver


def test_status_strings(lib):
    for code in range(7):
        s = lib.zeros_status_str(code).decode()
        assert s.startswith("ZEROS_"), s
    assert "unknown" in lib.zeros_status_str(99).decode()


def test_struct_layout_matches_header():
    assert ctypes.sizeof(L.zeros_shape) == 32
    assert ctypes.sizeof(L.zeros_state) == 8 * ctypes.sizeof(ctypes.c_void_p)


# placeholder addresses, far apart so they never overlap unless a test wants them to
P = {name: 0x10000000 * (i + 1) for i, name in enumerate(("q", "k", "v", "u", "mu", "tau", "g1", "gh", "o", "g0"))}


def shape(B=1, H=2, N=8, d=16, d_u=16, dtype=0, rope=0, base=10000.0):
    return L.zeros_shape(B, H, N, d, d_u, dtype, rope, base)


def call_causal(lib, shp, ptrs=None, state=None, state_in=None):
    p = dict(P, **(ptrs or {}))
    return lib.zeros_fwd_causal(ctypes.byref(shp) if shp is not None else None, p["q"], p["k"], p["v"],
                                p["u"], p["mu"], p["tau"], p["g1"], p["gh"], p["g0"], p["o"], state_in, state,
                                None, 0, None)


def call_encoder(lib, shp, ptrs=None, ws=None, ws_bytes=0):
    p = dict(P, **(ptrs or {}))
    return lib.zeros_fwd_encoder(ctypes.byref(shp), p["q"], p["k"], p["v"], p["u"], p["mu"], p["tau"],
                                 p["g1"], p["gh"], p["g0"], p["o"], ws, ws_bytes, None)


def call_decode(lib, shp, state, ptrs=None):
    p = dict(P, **(ptrs or {}))
    return lib.zeros_decode_step(ctypes.byref(shp), p["q"], p["k"], p["v"], p["u"], p["mu"], p["tau"],
                                 p["g1"], p["gh"], p["g0"], p["o"], state, None)


def test_null_shape(lib):
    assert call_causal(lib, None) == L.ZEROS_ERR_NULL
    assert "shape" in lib.zeros_last_error().decode()


@pytest.mark.parametrize("name", ["q", "k", "v", "u", "mu", "tau", "g1", "gh", "o"])
def test_null_tensor(lib, name):
    assert call_causal(lib, shape(), {name: None}) == L.ZEROS_ERR_NULL
    assert call_encoder(lib, shape(), {name: None}) == L.ZEROS_ERR_NULL


def test_bad_dtype(lib):
    assert call_causal(lib, shape(dtype=7)) == L.ZEROS_ERR_DTYPE


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=-1), dict(d=0), dict(d_u=0),
                                dict(B=1 << 20, H=1 << 10, N=1 << 10, d=128, d_u=128)])
def test_bad_sizes(lib, kw):
    assert call_causal(lib, shape(**kw)) == L.ZEROS_ERR_SHAPE


@pytest.mark.parametrize("kw", [dict(d=96, d_u=96), dict(d=256, d_u=256), dict(d=64, d_u=32),
                                dict(rope=2)])
def test_unsupported(lib, kw):
    assert call_causal(lib, shape(**kw)) == L.ZEROS_ERR_UNSUPPORTED


@pytest.mark.parametrize("base", [0.5, float("inf"), float("nan")])
def test_bad_rope_base(lib, base):
    assert call_causal(lib, shape(rope=1, base=base)) == L.ZEROS_ERR_SHAPE


def test_output_alias(lib):
    # o starts inside q's byte range: [B,H,N,d] = 1*2*8*16 f32 = 1024 bytes
    assert call_causal(lib, shape(), {"o": P["q"] + 512}) == L.ZEROS_ERR_ALIAS
    assert call_encoder(lib, shape(), {"o": P["gh"]}) == L.ZEROS_ERR_ALIAS
    assert call_decode(lib, shape(N=1), None, {"o": P["g0"]}) != L.ZEROS_OK
    assert call_encoder(lib, shape(), {"o": P["g0"]}) == L.ZEROS_ERR_ALIAS    # the optional gate too


def test_misaligned_tensors_rejected(lib):
    assert call_causal(lib, shape(), {"q": P["q"] + 2}) == L.ZEROS_ERR_SHAPE
    assert call_encoder(lib, shape(), {"o": P["o"] + 8}) == L.ZEROS_ERR_SHAPE


def test_workspace_size_and_validation(lib):
    bf = shape(B=2, H=16, N=16384, d=128, d_u=128, dtype=1)
    n = lib.zeros_fwd_causal_workspace_bytes(ctypes.byref(bf))
    bh, nch = 2 * 16, 16384 // 64
    logits = bh * 16384 * 4
    useg = bh * (16384 // 256) * 128 * 4
    agg = bh * nch * 16                                  # (max, sum e, sum s, pad) per 64-token chunk
    nseg = 8                                             # scan segments per head: 32 heads x 8 >= 256
    segsc = bh * nseg * 16                               # composed scalar map per segment
    segst = bh * (nseg - 1) * 3 * 128 * 128 * 4          # float32 X, Y, H per segment boundary
    sink = 64 * 128 * 2                                  # output rows past N of a last, partial chunk
    coef = bh * nch * (10 * 64 + 8) * 4                  # per-chunk scalar scan and coefficients
    assert n == logits + useg + agg + segsc + segst + sink + coef
    assert n < 80 << 20                                  # no per-chunk operand records in HBM
    # float32 path: logits [2, 8], u sums of one 256-token segment [2, 1, 16], aggregates of one
    # 64-token chunk [2, 1] float4, each region rounded up to 256 bytes
    assert lib.zeros_fwd_causal_workspace_bytes(ctypes.byref(shape(dtype=0))) == 3 * 256
    assert lib.zeros_fwd_causal_workspace_bytes(None) == 0
    small = shape(B=1, H=2, N=8, d=64, d_u=64, dtype=1)
    need = lib.zeros_fwd_causal_workspace_bytes(ctypes.byref(small))
    p = dict(P)
    r = lib.zeros_fwd_causal(ctypes.byref(small), p["q"], p["k"], p["v"], p["u"], p["mu"], p["tau"], p["g1"],
                             p["gh"], None, p["o"], None, None, 0x7000000, need - 1, None)
    assert r == L.ZEROS_ERR_SHAPE
    r = lib.zeros_fwd_causal(ctypes.byref(small), p["q"], p["k"], p["v"], p["u"], p["mu"], p["tau"], p["g1"],
                             p["gh"], None, p["o"], None, None, 0x7000010, need, None)
    assert r == L.ZEROS_ERR_SHAPE                                                       # misaligned


def test_library_never_allocates_scratch(lib):
    """Scratch comes from the caller: a call that needs a workspace and gets none is refused on the
    host (ZEROS_ERR_NULL, nothing launched), on both causal paths and for long bf16 encoders."""
    for shp in (shape(B=1, H=2, N=8, d=64, d_u=64, dtype=1), shape(dtype=0)):
        assert lib.zeros_fwd_causal_workspace_bytes(ctypes.byref(shp)) > 0
        assert call_causal(lib, shp) == L.ZEROS_ERR_NULL
        assert "workspace is NULL" in lib.zeros_last_error().decode()
    long_bf = shape(B=1, H=1, N=4097, d=64, d_u=64, dtype=1)
    need = lib.zeros_fwd_encoder_workspace_bytes(ctypes.byref(long_bf))
    assert need == long_encoder_ws(1, 1, 4097, 64)
    assert call_encoder(lib, long_bf) == L.ZEROS_ERR_NULL
    assert call_encoder(lib, long_bf, ws=0x7000000, ws_bytes=need - 1) == L.ZEROS_ERR_SHAPE
    assert call_encoder(lib, long_bf, ws=0x7000010, ws_bytes=need) == L.ZEROS_ERR_SHAPE   # misaligned


def long_encoder_ws(B, H, N, d):
    """Scratch of the token-parallel long encoder: per (b, h) the u sums of the 256-token blocks,
    the logits, and per state block (256 spb tokens, spb a power of two <= 8 that keeps about 512
    workgroups) its (max, sum, sum) and three float32 d x d partial states, then three bf16 states;
    each region rounded up to 256 bytes."""
    up = lambda x: (x + 255) // 256 * 256
    bh, nblk = B * H, (N + 255) // 256
    spb = 1
    while spb < 8 and bh * ((nblk + 2 * spb - 1) // (2 * spb)) >= 512:
        spb *= 2
    nsb = (nblk + spb - 1) // spb
    return (up(bh * nblk * d * 4) + up(bh * N * 4) + up(bh * nsb * 16) + up(bh * nsb * 3 * d * d * 4)
            + up(bh * 3 * d * d * 2))


def test_long_encoder_plan_sizes():
    """The state blocks grow while the grid keeps about 512 workgroups: 64 heads of 8192 tokens
    take 1024-token blocks (8 per head), one head keeps 256-token blocks."""
    d = 64
    part = 3 * d * d * 4
    assert long_encoder_ws(8, 8, 8192, d) == 64 * 32 * d * 4 + 64 * 8192 * 4 + 64 * 8 * 16 + 64 * 8 * part + 64 * 3 * d * d * 2
    assert long_encoder_ws(1, 1, 8192, d) == 32 * d * 4 + 8192 * 4 + 512 + 32 * part + 3 * d * d * 2


@pytest.mark.parametrize("kw,need", [
    (dict(B=2, H=3, N=767, d=128, d_u=128, dtype=1), 0),                     # one launch, logits in LDS
    (dict(B=2, H=3, N=768, d=128, d_u=128, dtype=1), long_encoder_ws(2, 3, 768, 128)),
    (dict(B=2, H=3, N=4097, d=128, d_u=128, dtype=1), long_encoder_ws(2, 3, 4097, 128)),
    (dict(B=2, H=3, N=9000, d=64, d_u=64, dtype=1), long_encoder_ws(2, 3, 9000, 64)),
    (dict(B=96, H=4, N=256, d=64, d_u=64, dtype=1), 0),                      # per-head variant
    (dict(B=96, H=4, N=257, d=64, d_u=64, dtype=1), long_encoder_ws(96, 4, 257, 64)),   # B H N d >= 96 Ki x 64
    (dict(B=64, H=4, N=300, d=64, d_u=64, dtype=1), 0),                      # B H N d < 96 Ki x 64
    (dict(B=32, H=4, N=400, d=128, d_u=128, dtype=1), long_encoder_ws(32, 4, 400, 128)),
    (dict(B=2, H=3, N=9000, d=64, d_u=64, dtype=0), 0),                      # float32 kernel
    (dict(B=2, H=3, N=9000, d=32, d_u=32, dtype=1), 0)])                     # VALU kernel
def test_encoder_workspace_bytes(lib, kw, need):
    """bfloat16 d 64/128 encoders take the token-parallel pipeline (and need scratch) from 768
    tokens, or from 257 tokens once q holds 96 Ki x 64 elements."""
    assert lib.zeros_fwd_encoder_workspace_bytes(ctypes.byref(shape(**kw))) == need


def test_noalloc_rejects_oversize_on_the_host(lib):
    """zeros_fwd_causal_noalloc refuses a call whose scratch exceeds its fixed array before any
    HIP call (placeholder pointers are never used)."""
    big = shape(B=1, H=64, N=262144, d=16, d_u=16, dtype=1)       # 16.8 M token-heads of logits alone
    assert lib.zeros_fwd_causal_workspace_bytes(ctypes.byref(big)) > (64 << 20)
    p = dict(P)
    r = lib.zeros_fwd_causal_noalloc(ctypes.byref(big), p["q"], p["k"], p["v"], p["u"], p["mu"], p["tau"],
                                     p["g1"], p["gh"], None, p["o"], None, None, None)
    assert r == L.ZEROS_ERR_UNSUPPORTED
    assert "more than the fixed" in lib.zeros_last_error().decode()
    assert lib.zeros_fwd_causal_noalloc(None, *([None] * 13)) == L.ZEROS_ERR_NULL


def test_partial_state_rejected(lib):
    st = L.zeros_state(1, 2, 3, 4, 5, 6, 7, None)
    assert call_causal(lib, shape(), state=ctypes.byref(st)) == L.ZEROS_ERR_NULL


def _aligned_state(base):
    return L.zeros_state(*(base + 0x100000 * i for i in range(8)))


def test_state_in_validation(lib):
    partial = L.zeros_state(1, 2, 3, 4, 5, 6, 7, None)
    assert call_causal(lib, shape(), state_in=ctypes.byref(partial)) == L.ZEROS_ERR_NULL
    mis = L.zeros_state(0x1000008, 0x2000000, 0x3000000, 0x4000000, 0x5000000, 0x6000000, 0x7000000, 0x8000000)
    assert call_causal(lib, shape(), state_in=ctypes.byref(mis)) == L.ZEROS_ERR_SHAPE
    a, b = _aligned_state(0xB0000000), _aligned_state(0xC0000000)      # away from the placeholders
    # the same state as input and output, or overlapping fields, is rejected
    assert call_causal(lib, shape(), state=ctypes.byref(a), state_in=ctypes.byref(a)) == L.ZEROS_ERR_ALIAS
    c = _aligned_state(0xC0000000)
    c.m = a.E
    assert call_causal(lib, shape(), state=ctypes.byref(c), state_in=ctypes.byref(a)) == L.ZEROS_ERR_ALIAS
    # o inside state_in's F
    assert call_causal(lib, shape(), {"o": a.F}, state=ctypes.byref(b), state_in=ctypes.byref(a)) == L.ZEROS_ERR_ALIAS


def test_written_state_must_not_overlap(lib):
    """A state the call writes (causal state_out, the decode state) may not overlap a tensor
    argument, o, or itself."""
    s = _aligned_state(0xB0000000)
    s.Su = P["q"]
    assert call_causal(lib, shape(), state=ctypes.byref(s)) == L.ZEROS_ERR_ALIAS
    s = _aligned_state(0xB0000000)
    s.t = P["o"]
    assert call_causal(lib, shape(), state=ctypes.byref(s)) == L.ZEROS_ERR_ALIAS
    assert call_decode(lib, shape(N=1), ctypes.byref(s)) == L.ZEROS_ERR_ALIAS
    s = _aligned_state(0xB0000000)
    s.G = s.F + 256                                   # F is 2 KiB at B1 H2 d16
    assert call_causal(lib, shape(), state=ctypes.byref(s)) == L.ZEROS_ERR_ALIAS
    assert call_decode(lib, shape(N=1), ctypes.byref(s)) == L.ZEROS_ERR_ALIAS
    s = _aligned_state(0xB0000000)
    s.m = P["g0"]
    assert call_decode(lib, shape(N=1), ctypes.byref(s)) == L.ZEROS_ERR_ALIAS


def test_decode_validation(lib):
    st = L.zeros_state(1, 2, 3, 4, 5, 6, 7, 8)
    assert call_decode(lib, shape(N=2), ctypes.byref(st)) == L.ZEROS_ERR_SHAPE
    assert call_decode(lib, shape(N=1), None) == L.ZEROS_ERR_NULL
    bad = L.zeros_state(1, 2, 3, None, 5, 6, 7, 8)
    assert call_decode(lib, shape(N=1), ctypes.byref(bad)) == L.ZEROS_ERR_NULL
    assert call_decode(lib, shape(N=1, d=48, d_u=48), ctypes.byref(st)) == L.ZEROS_ERR_UNSUPPORTED


def test_misaligned_state_rejected(lib):
    st = L.zeros_state(0x1000008, 0x2000000, 0x3000000, 0x4000000, 0x5000000, 0x6000000, 0x7000000, 0x8000000)
    assert call_decode(lib, shape(N=1), ctypes.byref(st)) == L.ZEROS_ERR_SHAPE
    assert call_causal(lib, shape(), state=ctypes.byref(st)) == L.ZEROS_ERR_SHAPE


def test_empty_sequence_is_a_noop(lib):
    none = {k: None for k in ("q", "k", "v", "u", "g1", "gh", "o")}
    assert call_causal(lib, shape(N=0), none) == L.ZEROS_OK
    assert call_encoder(lib, shape(N=0), none) == L.ZEROS_OK
    assert call_causal(lib, shape(N=0), {"mu": None}) == L.ZEROS_ERR_NULL
    assert call_causal(lib, shape(N=0)) == L.ZEROS_OK
    assert call_encoder(lib, shape(N=0)) == L.ZEROS_OK
    assert lib.zeros_last_error().decode() == ""


def test_state_bytes_and_packing(lib):
    S, H, d, du = 3, 5, 64, 64
    n = S * H
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    expect = 3 * a256(n * d * d * 4) + a256(n * du * 4) + 4 * a256(n * 4)
    assert lib.zeros_state_bytes(S, H, d, du) == expect
    assert lib.zeros_state_bytes(0, H, d, du) == 0
    st = L.zeros_state()
    base = 0x40000000
    assert lib.zeros_state_from_buffer(base, S, H, d, du, ctypes.byref(st)) == L.ZEROS_OK
    fields = [st.F, st.G, st.Hs, st.Su, st.m, st.E, st.P, st.t]
    assert fields[0] == base
    assert all(f % 256 == 0 for f in fields)
    assert fields == sorted(fields)
    assert st.t + n * 4 <= base + expect
    assert lib.zeros_state_from_buffer(None, S, H, d, du, ctypes.byref(st)) == L.ZEROS_ERR_NULL


def test_binding_arity_matches_header(lib):
    """The ctypes declarations of the binding take as many arguments as the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in ("zeros_fwd_causal", "zeros_fwd_encoder", "zeros_decode_step",
                 "zeros_fwd_causal_workspace_bytes", "zeros_fwd_encoder_workspace_bytes",
                 "zeros_fwd_causal_noalloc", "zeros_bwd_causal", "zeros_bwd_causal_workspace_bytes",
                 "zeros_state_bytes", "zeros_state_from_buffer"):
        m = re.search(r"\b%s\s*\(([^)]*)\)\s*;" % name, text)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(getattr(lib, name).argtypes) == len(params), name


def test_missing_library_fails_loudly():
    """No fallback: loading a library that is not there raises (in a fresh process, since the
    binding keeps the library it loaded)."""
    import subprocess
    import sys
    code = ("import zero_sum_attention_amd._lib as L\n"
            "try:\n    L.load_library('/nonexistent/libzeros.so')\n"
            "except ImportError as e:\n    print('raised', e)\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert "raised" in out.stdout and "not built" in out.stdout, out.stdout + out.stderr


def test_cpu_tensors_rejected():
    """The binding runs only the GPU library: CPU tensors are refused, nothing computes on the host."""
    import torch
    import zero_sum_attention_amd as Z
    q = torch.zeros(1, 1, 4, 16)
    g = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError, match="GPU"):
        Z.zeros_fwd_causal(q, q, q, q, torch.zeros(1, 16), torch.zeros(1), g, g)
    with pytest.raises(ValueError, match="GPU"):
        Z.zeros_fwd_encoder(q, q, q, q, torch.zeros(1, 16), torch.zeros(1), g, g)


@pytest.mark.parametrize("B,H,N,d,nseg", [(1, 2, 8192, 64, 64), (8, 8, 512, 64, 4), (1, 1, 1000, 128, 16),
                                          (64, 8, 512, 64, 1), (1, 1, 255, 16, 2), (1, 3, 577, 32, 4),
                                          (2, 2, 100, 16, 1)])
def test_float32_segment_plan_workspace(lib, B, H, N, d, nseg):
    """The float32 path's workspace carries segment states and carries exactly when the plan splits a
    head. Segments are whole 64-token blocks. d 64/128 (one workgroup per head segment): about one
    workgroup per CU, at most 64 segments, at least 64 tokens each. d 16/32 (one workgroup per
    16-column tile): at least 128 tokens each."""
    def up(x):
        return (x + 255) // 256 * 256
    bh = B * H
    expect = up(bh * N * 4) + up(bh * ((N + 255) // 256) * d * 4) + up(bh * ((N + 63) // 64) * 16)
    if nseg > 1:
        expect += up(bh * (nseg - 1) * 3 * d * d * 4) + up(bh * nseg * 4) + up(bh * nseg * 16)
    got = lib.zeros_fwd_causal_workspace_bytes(ctypes.byref(shape(B=B, H=H, N=N, d=d, d_u=d, dtype=0)))
    assert got == expect


# ---- ZeroS-SM (zeros_sm_fwd_causal): host-side validation only

def call_sm(lib, shp, ptrs=None, ws=None, ws_bytes=0):
    p = dict(P, **(ptrs or {}))
    return lib.zeros_sm_fwd_causal(ctypes.byref(shp) if shp is not None else None, p["q"], p["k"], p["v"],
                                   p["g1"], p["gh"], p["g0"], p["o"], ws, ws_bytes, None)


def sm_shape(**kw):
    base = dict(B=1, H=2, N=8, d=64, d_u=64, dtype=1)
    base.update(kw)
    return shape(**base)


def test_sm_rejects_bad_arguments(lib):
    assert call_sm(lib, None) == L.ZEROS_ERR_NULL
    for name in ("q", "k", "v", "g1", "gh", "o"):
        assert call_sm(lib, sm_shape(), {name: None}) == L.ZEROS_ERR_NULL
    assert call_sm(lib, sm_shape(dtype=0)) == L.ZEROS_ERR_UNSUPPORTED          # bfloat16 only
    assert call_sm(lib, sm_shape(dtype=7)) == L.ZEROS_ERR_DTYPE
    for d in (16, 32, 96, 256):
        assert call_sm(lib, sm_shape(d=d, d_u=d)) == L.ZEROS_ERR_UNSUPPORTED
    assert call_sm(lib, sm_shape(N=-1)) == L.ZEROS_ERR_SHAPE
    assert call_sm(lib, sm_shape(rope=1, base=0.5)) == L.ZEROS_ERR_SHAPE
    assert call_sm(lib, sm_shape(), {"q": P["q"] + 2}) == L.ZEROS_ERR_SHAPE  # misaligned
    assert call_sm(lib, sm_shape(), {"o": P["v"] + 256}) == L.ZEROS_ERR_ALIAS
    assert call_sm(lib, sm_shape(), {"o": P["g0"]}) == L.ZEROS_ERR_ALIAS
    # RoPE needs the workspace for the rotated q and k
    assert call_sm(lib, sm_shape(rope=1)) == L.ZEROS_ERR_NULL
    need = lib.zeros_sm_fwd_causal_workspace_bytes(ctypes.byref(sm_shape(rope=1)))
    assert need == 2 * 1 * 2 * 8 * 64 * 2
    assert call_sm(lib, sm_shape(rope=1), ws=0x7f000000, ws_bytes=need - 1) == L.ZEROS_ERR_SHAPE
    assert call_sm(lib, sm_shape(rope=1), ws=P["q"], ws_bytes=need) == L.ZEROS_ERR_ALIAS
    assert lib.zeros_sm_fwd_causal_workspace_bytes(ctypes.byref(sm_shape())) == 0
    # no tokens: nothing to do, whatever the pointers
    assert call_sm(lib, sm_shape(N=0), {"q": None, "o": None}) == L.ZEROS_OK
