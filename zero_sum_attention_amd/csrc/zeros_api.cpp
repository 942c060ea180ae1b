// C-ABI front end of libzeros: argument validation, dispatch and error reporting.
// Every check runs on the host before any HIP call, so invalid arguments never reach a kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>

#include "launch.hpp"

// Fixed scratch of zeros_fwd_causal_noalloc: one copy per device, held until the process ends.
// Host code never uses its name as an address (on the host it is only a stand-in): the device
// address comes from hipGetSymbolAddress, once per device with that device current, and is kept
// per device.
static __device__ __align__(256) unsigned char scratch[ZEROS_NOALLOC_SCRATCH_BYTES];

namespace {
// The matrix-core path covers bfloat16 inputs with d in {64, 128}; everything else (float32
// inputs, small heads) runs on the float32 VALU kernel.
bool causal_uses_mfma(const zeros_shape *s) {
    return s->dtype == ZEROS_BF16 && (s->d == 64 || s->d == 128);
}
}  // namespace

namespace {

thread_local std::string g_last_error;

zeros_status fail(zeros_status st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

zeros_status ok() {
    g_last_error.clear();
    return ZEROS_OK;
}

size_t elem_bytes(int dtype) { return dtype == ZEROS_BF16 ? 2 : 4; }

struct Range {
    const void *p;
    size_t bytes;
};

bool overlap(const Range &a, const Range &b) {
    if (a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Common validation of the shape and the input/output pointers. `tokens` is the number of
// token rows per (b, h) that the call reads (N for the forward calls, 1 for decode).
zeros_status check_common(const zeros_shape *s, const void *q, const void *k, const void *v,
                          const void *u, const float *mu, const float *tau, const void *g1,
                          const void *gh, const void *g0, const void *o, const char *fn) {
    const std::string f(fn);
    if (!s) return fail(ZEROS_ERR_NULL, f + ": shape is NULL");
    if (!mu || !tau) return fail(ZEROS_ERR_NULL, f + ": mu or tau is NULL");
    // token tensors may be NULL only when there are no tokens (N = 0)
    if ((!q || !k || !v || !u || !g1 || !gh || !o) && s->N != 0)
        return fail(ZEROS_ERR_NULL, f + ": a tensor pointer is NULL");
    if (s->dtype != ZEROS_F32 && s->dtype != ZEROS_BF16)
        return fail(ZEROS_ERR_DTYPE, f + ": dtype must be ZEROS_F32 or ZEROS_BF16");
    if (s->B < 1 || s->H < 1 || s->N < 0 || s->d < 1 || s->d_u < 1)
        return fail(ZEROS_ERR_SHAPE, f + ": need B, H, d, d_u >= 1 and N >= 0");
    if (s->d != 16 && s->d != 32 && s->d != 64 && s->d != 128)
        return fail(ZEROS_ERR_UNSUPPORTED, f + ": d must be 16, 32, 64 or 128");
    if (s->d_u != s->d) return fail(ZEROS_ERR_UNSUPPORTED, f + ": d_u must equal d");
    if (s->rope != 0 && s->rope != 1) return fail(ZEROS_ERR_UNSUPPORTED, f + ": rope must be 0 or 1");
    if (s->rope == 1 && !(std::isfinite(s->rope_base) && s->rope_base > 1.0f))
        return fail(ZEROS_ERR_SHAPE, f + ": rope_base must be finite and > 1");
    const long double elems = static_cast<long double>(s->B) * s->H * s->N * s->d;
    if (elems >= 2147483648.0L) return fail(ZEROS_ERR_SHAPE, f + ": tensor has 2^31 elements or more");
    const size_t eb = elem_bytes(s->dtype);
    const size_t tens = static_cast<size_t>(s->B) * s->H * s->N * s->d * eb;
    const size_t gate = static_cast<size_t>(s->B) * s->H * s->N * eb;
    auto al16 = [](const void *x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; };
    if (s->N != 0 && !(al16(q) && al16(k) && al16(v) && al16(u) && al16(o)))
        return fail(ZEROS_ERR_SHAPE, f + ": q, k, v, u and o must be 16-byte aligned");
    const Range out{o, tens};
    const Range ins[] = {{q, tens}, {k, tens}, {v, tens}, {u, tens}, {g1, gate}, {gh, gate},
                         {g0, g0 ? gate : 0},
                         {mu, static_cast<size_t>(s->H) * s->d_u * 4}, {tau, static_cast<size_t>(s->H) * 4}};
    for (const Range &r : ins)
        if (overlap(out, r)) return fail(ZEROS_ERR_ALIAS, f + ": o overlaps an input");
    return ZEROS_OK;
}

bool state_complete(const zeros_state *st) {
    return st->F && st->G && st->Hs && st->Su && st->m && st->E && st->P && st->t;
}

// The state matrices are streamed with 16-byte accesses; the scalars need 4-byte alignment.
bool state_aligned(const zeros_state *st) {
    auto al = [](const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
    return al(st->F, 16) && al(st->G, 16) && al(st->Hs, 16) && al(st->Su, 4) && al(st->m, 4) &&
           al(st->E, 4) && al(st->P, 4) && al(st->t, 4);
}

// Byte ranges of the fields of a state of S x H heads (for the overlap checks).
void state_ranges(const zeros_state *st, const zeros_shape *s, Range (&r)[8]) {
    const size_t n = static_cast<size_t>(s->B) * s->H;
    const size_t mat = n * s->d * s->d * 4;
    r[0] = {st->F, mat}; r[1] = {st->G, mat}; r[2] = {st->Hs, mat};
    r[3] = {st->Su, n * s->d_u * 4}; r[4] = {st->m, n * 4}; r[5] = {st->E, n * 4};
    r[6] = {st->P, n * 4}; r[7] = {st->t, n * 4};
}

// A state the call writes must not overlap the call's inputs, its output or itself.
zeros_status check_written_state(const zeros_state *st, const zeros_shape *s, const void *q, const void *k,
                                 const void *v, const void *u, const float *mu, const float *tau,
                                 const void *g1, const void *gh, const void *g0, const void *o,
                                 const char *fn) {
    const size_t eb = elem_bytes(s->dtype);
    const size_t tens = static_cast<size_t>(s->B) * s->H * s->N * s->d * eb;
    const size_t gate = static_cast<size_t>(s->B) * s->H * s->N * eb;
    const Range io[] = {{q, tens}, {k, tens}, {v, tens}, {u, tens}, {g1, gate}, {gh, gate},
                        {g0, g0 ? gate : 0}, {o, tens},
                        {mu, static_cast<size_t>(s->H) * s->d_u * 4}, {tau, static_cast<size_t>(s->H) * 4}};
    Range r[8];
    state_ranges(st, s, r);
    for (int i = 0; i < 8; ++i) {
        for (const Range &x : io)
            if (overlap(r[i], x)) return fail(ZEROS_ERR_ALIAS, std::string(fn) + ": the written state overlaps a tensor argument");
        for (int j = 0; j < i; ++j)
            if (overlap(r[i], r[j])) return fail(ZEROS_ERR_ALIAS, std::string(fn) + ": fields of the written state overlap");
    }
    return ZEROS_OK;
}

zeros::Problem make_problem(const zeros_shape *s, const void *q, const void *k, const void *v,
                            const void *u, const float *mu, const float *tau, const void *g1,
                            const void *gh, const void *g0, void *o, const zeros_state *st) {
    zeros::Problem p{};
    p.q = q; p.k = k; p.v = v; p.u = u; p.mu = mu; p.tau = tau; p.g1 = g1; p.gh = gh; p.o = o;
    p.g0 = s->N != 0 ? g0 : nullptr;
    if (st) p.st = *st;
    p.B = s->B; p.H = s->H; p.N = s->N; p.d = s->d; p.du = s->d_u;
    p.dtype = s->dtype; p.rope = s->rope; p.rope_base = s->rope_base;
    return p;
}

zeros_status hip_result(hipError_t err, const char *fn) {
    if (err != hipSuccess)
        return fail(ZEROS_ERR_HIP, std::string(fn) + ": " + hipGetErrorName(err) + ": " + hipGetErrorString(err));
    return ok();
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The library allocates nothing: scratch comes from the caller. `need` = 0 accepts any workspace
// (including NULL).
zeros_status check_workspace(const void *ws, size_t bytes, size_t need, const char *fn) {
    if (need == 0) return ZEROS_OK;
    if (!ws)
        return fail(ZEROS_ERR_NULL, std::string(fn) + ": workspace is NULL but this call needs " + std::to_string(need) +
                                        " bytes of scratch (see the *_workspace_bytes query)");
    if (bytes < need) return fail(ZEROS_ERR_SHAPE, std::string(fn) + ": workspace smaller than the *_workspace_bytes query");
    if (reinterpret_cast<uintptr_t>(ws) & 255u)
        return fail(ZEROS_ERR_SHAPE, std::string(fn) + ": workspace must be 256-byte aligned");
    return ZEROS_OK;
}

// Validation shared by the causal entry points. On success `noop` tells whether the call has
// nothing to do (N = 0 without a state to write); otherwise `p` is the problem, `mfma` the path
// it takes and `need` the scratch bytes of that path.
zeros_status causal_prepare(const char *fn, const zeros_shape *shape, const void *q, const void *k,
                            const void *v, const void *u, const float *mu, const float *tau, const void *g1,
                            const void *gh, const void *g0, void *o, const zeros_state *state_in,
                            const zeros_state *state_out, zeros::Problem &p, bool &mfma, size_t &need,
                            bool &noop) {
    const std::string f(fn);
    zeros_status st = check_common(shape, q, k, v, u, mu, tau, g1, gh, g0, o, fn);
    if (st != ZEROS_OK) return st;
    if (state_in && !state_complete(state_in)) return fail(ZEROS_ERR_NULL, f + ": a state_in field is NULL");
    if (state_in && !state_aligned(state_in))
        return fail(ZEROS_ERR_SHAPE, f + ": state_in matrices must be 16-byte aligned");
    if (state_out && !state_complete(state_out)) return fail(ZEROS_ERR_NULL, f + ": a state_out field is NULL");
    if (state_out && !state_aligned(state_out))
        return fail(ZEROS_ERR_SHAPE, f + ": state_out matrices must be 16-byte aligned");
    if (state_out) {
        st = check_written_state(state_out, shape, q, k, v, u, mu, tau, g1, gh, g0, o, fn);
        if (st != ZEROS_OK) return st;
    }
    if (state_in && state_out) {
        Range a[8], b[8];
        state_ranges(state_in, shape, a);
        state_ranges(state_out, shape, b);
        for (const Range &x : a)
            for (const Range &y : b)
                if (overlap(x, y)) return fail(ZEROS_ERR_ALIAS, f + ": state_out overlaps state_in");
    }
    if (state_in && shape->N != 0) {
        Range a[8];
        state_ranges(state_in, shape, a);
        const Range out{o, static_cast<size_t>(shape->B) * shape->H * shape->N * shape->d * elem_bytes(shape->dtype)};
        for (const Range &x : a)
            if (overlap(x, out)) return fail(ZEROS_ERR_ALIAS, f + ": o overlaps state_in");
    }
    noop = shape->N == 0 && !state_out;
    if (noop) return ZEROS_OK;
    p = make_problem(shape, q, k, v, u, mu, tau, g1, gh, g0, o, state_out);
    if (state_in) p.sin = *state_in;
    // a continued empty call (a copy of the state) takes the float32 path
    mfma = causal_uses_mfma(shape) && !(state_in && shape->N == 0);
    need = mfma ? zeros::causal_work_bytes(shape->B, shape->H, shape->N, shape->d_u)
                : zeros::causal_valu_work_bytes(shape->B, shape->H, shape->N, shape->d_u);
    return ZEROS_OK;
}

hipError_t causal_launch(const zeros::Problem &p, bool mfma, void *ws, hipStream_t hs) {
    return mfma ? zeros::launch_causal_mfma(p, zeros::causal_work_carve(ws, p.B, p.H, p.N, p.du), hs)
                : zeros::launch_causal_valu(p, zeros::causal_valu_work_carve(ws, p.B, p.H, p.N, p.du), hs);
}

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array.
zeros_status scratch_for_current_device(void **ptr, const char *fn) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_result(err, fn);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(ZEROS_ERR_UNSUPPORTED, std::string(fn) + ": device index beyond the supported 64");
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // two threads may both resolve it on a first call; they store the same address
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return hip_result(err, fn);
        if (!p) return fail(ZEROS_ERR_HIP, std::string(fn) + ": hipGetSymbolAddress returned NULL");
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return ZEROS_OK;
}

}  // namespace

extern "C" {

zeros_status zeros_fwd_causal(const zeros_shape *shape, const void *q, const void *k, const void *v,
                              const void *u, const float *mu, const float *tau, const void *g1,
                              const void *gh, const void *g0, void *o, const zeros_state *state_in,
                              const zeros_state *state_out, void *workspace, size_t workspace_bytes,
                              void *stream) {
    zeros::Problem p{};
    bool mfma = false, noop = false;
    size_t need = 0;
    zeros_status st = causal_prepare("zeros_fwd_causal", shape, q, k, v, u, mu, tau, g1, gh, g0, o, state_in,
                                     state_out, p, mfma, need, noop);
    if (st != ZEROS_OK) return st;
    if (noop) return ok();
    st = check_workspace(workspace, workspace_bytes, need, "zeros_fwd_causal");
    if (st != ZEROS_OK) return st;
    return hip_result(causal_launch(p, mfma, workspace, static_cast<hipStream_t>(stream)), "zeros_fwd_causal");
}

zeros_status zeros_fwd_causal_noalloc(const zeros_shape *shape, const void *q, const void *k, const void *v,
                                      const void *u, const float *mu, const float *tau, const void *g1,
                                      const void *gh, const void *g0, void *o, const zeros_state *state_in,
                                      const zeros_state *state_out, void *stream) {
    const char *fn = "zeros_fwd_causal_noalloc";
    zeros::Problem p{};
    bool mfma = false, noop = false;
    size_t need = 0;
    zeros_status st = causal_prepare(fn, shape, q, k, v, u, mu, tau, g1, gh, g0, o, state_in, state_out, p, mfma,
                                     need, noop);
    if (st != ZEROS_OK) return st;
    if (noop) return ok();
    if (need > static_cast<size_t>(ZEROS_NOALLOC_SCRATCH_BYTES))
        return fail(ZEROS_ERR_UNSUPPORTED, std::string(fn) + ": this call needs " + std::to_string(need) +
                                               " bytes of scratch, more than the fixed " +
                                               std::to_string(static_cast<size_t>(ZEROS_NOALLOC_SCRATCH_BYTES)) +
                                               " (use zeros_fwd_causal with a workspace)");
    void *ws = nullptr;
    st = scratch_for_current_device(&ws, fn);
    if (st != ZEROS_OK) return st;
    return hip_result(causal_launch(p, mfma, ws, static_cast<hipStream_t>(stream)), fn);
}

size_t zeros_fwd_causal_workspace_bytes(const zeros_shape *shape) {
    if (!shape || shape->B < 1 || shape->H < 1 || shape->N < 0 || shape->d_u < 1) return 0;
    const size_t valu = zeros::causal_valu_work_bytes(shape->B, shape->H, shape->N, shape->d_u);
    if (!causal_uses_mfma(shape)) return valu;
    // a call continued from a state with N = 0 (a copy of the state) takes the float32 path;
    // every other call of this shape takes the matrix-core path: cover both
    return std::max(valu, zeros::causal_work_bytes(shape->B, shape->H, shape->N, shape->d_u));
}

zeros_status zeros_fwd_encoder(const zeros_shape *shape, const void *q, const void *k, const void *v,
                               const void *u, const float *mu, const float *tau, const void *g1,
                               const void *gh, const void *g0, void *o, void *workspace,
                               size_t workspace_bytes, void *stream) {
    zeros_status st = check_common(shape, q, k, v, u, mu, tau, g1, gh, g0, o, "zeros_fwd_encoder");
    if (st != ZEROS_OK) return st;
    if (shape->N == 0) return ok();
    const zeros::Problem p = make_problem(shape, q, k, v, u, mu, tau, g1, gh, g0, o, nullptr);
    st = check_workspace(workspace, workspace_bytes, zeros::encoder_work_bytes(p), "zeros_fwd_encoder");
    if (st != ZEROS_OK) return st;
    return hip_result(zeros::launch_encoder(p, workspace, static_cast<hipStream_t>(stream)), "zeros_fwd_encoder");
}

size_t zeros_fwd_encoder_workspace_bytes(const zeros_shape *shape) {
    if (!shape || shape->B < 1 || shape->H < 1 || shape->N < 0 || shape->d < 1 || shape->d_u < 1) return 0;
    zeros::Problem p{};
    p.B = shape->B; p.H = shape->H; p.N = shape->N; p.d = shape->d; p.du = shape->d_u;
    p.dtype = shape->dtype;
    return zeros::encoder_work_bytes(p);
}

namespace {
// Validation of a ZeroS-SM call (no u, mu, tau; bfloat16 with d 64 or 128 only).
zeros_status sm_check(const zeros_shape *s, const void *q, const void *k, const void *v, const void *g1,
                      const void *gh, const void *g0, const void *o, const char *fn) {
    const std::string f(fn);
    if (!s) return fail(ZEROS_ERR_NULL, f + ": shape is NULL");
    if ((!q || !k || !v || !g1 || !gh || !o) && s->N != 0) return fail(ZEROS_ERR_NULL, f + ": a tensor pointer is NULL");
    if (s->dtype != ZEROS_F32 && s->dtype != ZEROS_BF16)
        return fail(ZEROS_ERR_DTYPE, f + ": dtype must be ZEROS_F32 or ZEROS_BF16");
    if (s->B < 1 || s->H < 1 || s->N < 0 || s->d < 1 || s->d_u < 1)
        return fail(ZEROS_ERR_SHAPE, f + ": need B, H, d, d_u >= 1 and N >= 0");
    if (s->dtype != ZEROS_BF16) return fail(ZEROS_ERR_UNSUPPORTED, f + ": only bfloat16 inputs are supported");
    if (s->d != 64 && s->d != 128) return fail(ZEROS_ERR_UNSUPPORTED, f + ": d must be 64 or 128");
    if (s->rope != 0 && s->rope != 1) return fail(ZEROS_ERR_UNSUPPORTED, f + ": rope must be 0 or 1");
    if (s->rope == 1 && !(std::isfinite(s->rope_base) && s->rope_base > 1.0f))
        return fail(ZEROS_ERR_SHAPE, f + ": rope_base must be finite and > 1");
    const long double elems = static_cast<long double>(s->B) * s->H * s->N * s->d;
    if (elems >= 2147483648.0L) return fail(ZEROS_ERR_SHAPE, f + ": tensor has 2^31 elements or more");
    auto al16 = [](const void *x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; };
    if (s->N != 0 && !(al16(q) && al16(k) && al16(v) && al16(o)))
        return fail(ZEROS_ERR_SHAPE, f + ": q, k, v and o must be 16-byte aligned");
    const size_t tens = static_cast<size_t>(s->B) * s->H * s->N * s->d * 2;
    const size_t gate = static_cast<size_t>(s->B) * s->H * s->N * 2;
    const Range out{o, tens};
    const Range ins[] = {{q, tens}, {k, tens}, {v, tens}, {g1, gate}, {gh, gate}, {g0, g0 ? gate : 0}};
    for (const Range &r : ins)
        if (overlap(out, r)) return fail(ZEROS_ERR_ALIAS, f + ": o overlaps an input");
    return ZEROS_OK;
}

zeros::Problem sm_problem(const zeros_shape *s, const void *q, const void *k, const void *v, const void *g1,
                          const void *gh, const void *g0, void *o) {
    zeros::Problem p{};
    p.q = q; p.k = k; p.v = v; p.g1 = g1; p.gh = gh; p.g0 = s->N != 0 ? g0 : nullptr; p.o = o;
    p.B = s->B; p.H = s->H; p.N = s->N; p.d = s->d; p.du = s->d_u;
    p.dtype = s->dtype; p.rope = s->rope; p.rope_base = s->rope_base;
    return p;
}
}  // namespace

zeros_status zeros_sm_fwd_causal(const zeros_shape *shape, const void *q, const void *k, const void *v,
                                 const void *g1, const void *gh, const void *g0, void *o, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    const char *fn = "zeros_sm_fwd_causal";
    zeros_status st = sm_check(shape, q, k, v, g1, gh, g0, o, fn);
    if (st != ZEROS_OK) return st;
    if (shape->N == 0) return ok();
    const zeros::Problem p = sm_problem(shape, q, k, v, g1, gh, g0, o);
    st = check_workspace(workspace, workspace_bytes, zeros::sm_work_bytes(p), fn);
    if (st != ZEROS_OK) return st;
    if (workspace) {
        // the rotated q and k are written there: it must not overlap the inputs or o
        const size_t tens = static_cast<size_t>(p.B) * p.H * p.N * p.d * 2;
        const Range wr{workspace, zeros::sm_work_bytes(p)};
        const Range io[] = {{q, tens}, {k, tens}, {v, tens}, {o, tens}};
        for (const Range &r : io)
            if (overlap(wr, r)) return fail(ZEROS_ERR_ALIAS, std::string(fn) + ": workspace overlaps a tensor argument");
    }
    return hip_result(zeros::launch_sm_causal(p, workspace, static_cast<hipStream_t>(stream)), fn);
}

size_t zeros_sm_fwd_causal_workspace_bytes(const zeros_shape *shape) {
    if (!shape || shape->B < 1 || shape->H < 1 || shape->N < 0 || shape->d < 1) return 0;
    zeros::Problem p{};
    p.B = shape->B; p.H = shape->H; p.N = shape->N; p.d = shape->d; p.rope = shape->rope == 1;
    return zeros::sm_work_bytes(p);
}

zeros_status zeros_decode_step(const zeros_shape *shape, const void *q, const void *k, const void *v,
                               const void *u, const float *mu, const float *tau, const void *g1,
                               const void *gh, const void *g0, void *o, const zeros_state *state,
                               void *stream) {
    zeros_status st = check_common(shape, q, k, v, u, mu, tau, g1, gh, g0, o, "zeros_decode_step");
    if (st != ZEROS_OK) return st;
    if (shape->N != 1) return fail(ZEROS_ERR_SHAPE, "zeros_decode_step: N must be 1");
    if (!state) return fail(ZEROS_ERR_NULL, "zeros_decode_step: state is NULL");
    if (!state_complete(state)) return fail(ZEROS_ERR_NULL, "zeros_decode_step: a state field is NULL");
    if (!state_aligned(state))
        return fail(ZEROS_ERR_SHAPE, "zeros_decode_step: state matrices must be 16-byte aligned");
    st = check_written_state(state, shape, q, k, v, u, mu, tau, g1, gh, g0, o, "zeros_decode_step");
    if (st != ZEROS_OK) return st;
    const zeros::Problem p = make_problem(shape, q, k, v, u, mu, tau, g1, gh, g0, o, state);
    return hip_result(zeros::launch_decode(p, static_cast<hipStream_t>(stream)), "zeros_decode_step");
}

zeros_status zeros_bwd_causal(const zeros_shape *shape, const void *q, const void *k, const void *v,
                              const void *u, const float *mu, const float *tau, const void *g1,
                              const void *gh, const void *g0, const void *dO, void *dq, void *dk, void *dv,
                              void *du, float *dmu, float *dtau, void *dg1, void *dgh, void *dg0,
                              void *workspace, size_t workspace_bytes, void *stream) {
    const char *fn = "zeros_bwd_causal";
    const std::string f(fn);
    zeros_status st = check_common(shape, q, k, v, u, mu, tau, g1, gh, g0, dq, fn);
    if (st != ZEROS_OK) return st;
    const bool empty = shape->N == 0;
    if (!dmu || !dtau) return fail(ZEROS_ERR_NULL, f + ": dmu or dtau is NULL");
    if (!empty && (!dO || !dk || !dv || !du || !dg1 || !dgh))
        return fail(ZEROS_ERR_NULL, f + ": a gradient pointer is NULL");
    if (!empty && (g0 != nullptr) != (dg0 != nullptr))
        return fail(ZEROS_ERR_NULL, f + ": dg0 must be given exactly when g0 is");
    auto al16 = [](const void *x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; };
    if (!empty && !(al16(dO) && al16(dk) && al16(dv) && al16(du)))
        return fail(ZEROS_ERR_SHAPE, f + ": dO, dq, dk, dv and du must be 16-byte aligned");
    auto al4 = [](const void *x) { return (reinterpret_cast<uintptr_t>(x) & 3u) == 0; };
    if (!al4(dmu) || !al4(dtau)) return fail(ZEROS_ERR_SHAPE, f + ": dmu and dtau must be 4-byte aligned");
    const size_t eb = elem_bytes(shape->dtype);
    const size_t tens = static_cast<size_t>(shape->B) * shape->H * shape->N * shape->d * eb;
    const size_t gate = static_cast<size_t>(shape->B) * shape->H * shape->N * eb;
    const size_t mub = static_cast<size_t>(shape->H) * shape->d_u * 4, taub = static_cast<size_t>(shape->H) * 4;
    const Range ins[] = {{q, tens}, {k, tens}, {v, tens}, {u, tens}, {g1, gate}, {gh, gate},
                         {g0, g0 ? gate : 0}, {dO, tens}, {mu, mub}, {tau, taub}};
    const Range outs[] = {{dq, tens}, {dk, tens}, {dv, tens}, {du, tens}, {dg1, gate}, {dgh, gate},
                          {dg0, dg0 ? gate : 0}, {dmu, mub}, {dtau, taub}};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Range &r : ins)
            if (overlap(outs[i], r)) return fail(ZEROS_ERR_ALIAS, f + ": a gradient overlaps an input");
        for (size_t j = 0; j < i; ++j)
            if (overlap(outs[i], outs[j])) return fail(ZEROS_ERR_ALIAS, f + ": two gradients overlap");
    }
    const size_t need = zeros::causal_bwd_work_bytes(shape->B, shape->H, shape->N, shape->d);
    st = check_workspace(workspace, workspace_bytes, need, fn);
    if (st != ZEROS_OK) return st;
    const zeros::Problem p = make_problem(shape, q, k, v, u, mu, tau, g1, gh, g0, nullptr, nullptr);
    const zeros::BwdGrads g{dO, dq, dk, dv, du, dmu, dtau, dg1, dgh, g0 ? dg0 : nullptr};
    const zeros::BwdWork w = zeros::causal_bwd_work_carve(workspace, shape->B, shape->H, shape->N, shape->d);
    return hip_result(zeros::launch_causal_bwd(p, g, w, static_cast<hipStream_t>(stream)), fn);
}

size_t zeros_bwd_causal_workspace_bytes(const zeros_shape *shape) {
    if (!shape || shape->B < 1 || shape->H < 1 || shape->N < 0) return 0;
    if (shape->d != 16 && shape->d != 32 && shape->d != 64 && shape->d != 128) return 0;
    return zeros::causal_bwd_work_bytes(shape->B, shape->H, shape->N, shape->d);
}

size_t zeros_state_bytes(int32_t S, int32_t H, int32_t d, int32_t d_u) {
    if (S < 1 || H < 1 || d < 1 || d_u < 1) return 0;
    const long double heads = static_cast<long double>(S) * H;
    if (heads * (3.0L * d * d + d_u + 4.0L) * 4.0L >= 9.0e18L) return 0;
    const size_t n = static_cast<size_t>(S) * H;
    const size_t mat = align256(n * d * d * 4);
    return 3 * mat + align256(n * d_u * 4) + 4 * align256(n * 4);
}

zeros_status zeros_state_from_buffer(void *base, int32_t S, int32_t H, int32_t d, int32_t d_u,
                                     zeros_state *out) {
    if (!base || !out) return fail(ZEROS_ERR_NULL, "zeros_state_from_buffer: NULL argument");
    if (zeros_state_bytes(S, H, d, d_u) == 0) return fail(ZEROS_ERR_SHAPE, "zeros_state_from_buffer: bad sizes");
    const size_t n = static_cast<size_t>(S) * H;
    const size_t mat = align256(n * d * d * 4), vec = align256(n * d_u * 4), sc = align256(n * 4);
    char *b = static_cast<char *>(base);
    out->F = reinterpret_cast<float *>(b);
    out->G = reinterpret_cast<float *>(b + mat);
    out->Hs = reinterpret_cast<float *>(b + 2 * mat);
    out->Su = reinterpret_cast<float *>(b + 3 * mat);
    out->m = reinterpret_cast<float *>(b + 3 * mat + vec);
    out->E = reinterpret_cast<float *>(b + 3 * mat + vec + sc);
    out->P = reinterpret_cast<float *>(b + 3 * mat + vec + 2 * sc);
    out->t = reinterpret_cast<int32_t *>(b + 3 * mat + vec + 3 * sc);
    return ok();
}

const char *zeros_status_str(int32_t status) {
    switch (status) {
        case ZEROS_OK: return "ZEROS_OK: success";
        case ZEROS_ERR_NULL: return "ZEROS_ERR_NULL: a required pointer is NULL";
        case ZEROS_ERR_SHAPE: return "ZEROS_ERR_SHAPE: invalid sizes";
        case ZEROS_ERR_DTYPE: return "ZEROS_ERR_DTYPE: unknown dtype";
        case ZEROS_ERR_UNSUPPORTED: return "ZEROS_ERR_UNSUPPORTED: valid but not implemented";
        case ZEROS_ERR_HIP: return "ZEROS_ERR_HIP: HIP runtime error";
        case ZEROS_ERR_ALIAS: return "ZEROS_ERR_ALIAS: output overlaps an input";
        default: return "unknown zeros_status";
    }
}

const char *zeros_last_error(void) { return g_last_error.c_str(); }

int32_t zeros_abi_version(void) { return ZEROS_ABI_VERSION; }

}  // extern "C"
