// Causal ZeroS forward on the matrix cores: bfloat16 q/k/v with float32 states, d in {64, 128}.
//
// Method: Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计
// (zero-sum weights w_{t,i} = alpha_t e^{s_i} + beta_t s_i + gamma_t after expanding the gated
// first-order and residual terms; angular factor q^_t . k^_i with RoPE as a relative rotation;
// the prefix states of the linear-time scan). The optional zero-order gate of the same section
// (a first layer may keep the uniform term) adds sigma0_t/t to gamma_t. The logits s_i and
// per-chunk logit aggregates come from logits.hip. The sequence is cut into chunks of kC = 64
// tokens.
//
// causal_scan_kernel, one workgroup of d/16 waves per (batch, head, segment of the chunks), walks
//   its chunks in order; wave w owns value columns [16w, 16w+16) and all d rows of X, Y, H in
//   float32 registers. Per chunk, in LDS only:
//   (1) every thread takes 16 features of one token row of the raw q and k (copied into LDS by
//       direct global-to-LDS loads during the previous chunk) to unit, RoPE-rotated q^ and k^
//       rows in bf16; wave 0 runs the chunk's scalar scan and coefficients from the logit carry;
//   (2) the waves build k^T as MFMA A-operands and A^T = K Q^T on MFMA, turned into the
//       intra-chunk weights W_{t,i} = A (a_t e^{s_i-m_t} + b_t s_i + g_t), i <= t, as B-operands;
//   (3) each wave: o^T = S^T Q^T (carried states, S^T straight from the registers) + V^T W^T
//       (intra-chunk), then the states advance to the chunk end with K^T V' on MFMA. The W
//       accumulator layout is the B-operand layout of V^T W^T up to a permutation of the
//       contraction index, which V^T is read with.
//   Segments are chained exactly by a pass over each segment from a zero state (the same kernel
//   without queries and outputs) and a combine step (see the segment-parallel scan below).
// States are kept in a centred basis, X = F/E - H/t0 and Y = G - (P/t0) H. Both have zero-sum
// weights, so they stay of the size of the output, and rounding them (and the update operands)
// to bfloat16 for the MFMA is not amplified by the cancellation between alpha F, beta G and
// gamma H. With RoPE, q^ and k^ are rotated by their absolute position (the phase of the chunk
// start, reduced in double precision, plus the in-chunk offset times the frequency, in
// revolutions for the hardware sine and cosine), so the carried states are in the absolute frame
// and need no re-basing between chunks.
#include <hip/hip_bf16.h>

#include "device_common.hpp"
#include "kv_states.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace zeros {
namespace {

constexpr int kC = 64;          // tokens per chunk
constexpr int kTile = 16;       // value columns per workgroup
constexpr int kPad = 8;         // bf16 elements of row padding in LDS

// Order of the keys along the contraction index of every K^T V-type product in a 32-key block:
// lane group g4 holds keys {4 g4 + [0, 4)} and {16 + 4 g4 + [0, 4)}, which is the order the
// intra-chunk weights W come in from the A^T tiles (each tile gives a lane 4 keys). The staged v
// operands are stored in this order, so the same 16 bytes serve the state update and V^T W^T.
__device__ __forceinline__ int kperm(int key) {
    return (key & ~31) | (((key & 15) >> 2) << 3) | (((key >> 4) & 1) << 2) | (key & 3);
}

// (max, sum e^{s-max}) combine of two partial scans; a max of -inf marks an empty part.
__device__ __forceinline__ void lse_combine(float &m, float &e, float m2, float e2) {
    if (m2 == kNegInf) return;
    if (m == kNegInf) { m = m2; e = e2; return; }
    if (m >= m2) {
        e += e2 * __expf(m2 - m);
    } else {
        e = e * __expf(m - m2) + e2;
        m = m2;
    }
}

// Scalar scan of one chunk (one wave; lane r = token t0 + r + 1) and its coefficients.
// Inputs: the chunk's logits and gate pre-activations in lanes (s0 = sigma0 of the optional
// zero-order gate, 0 without it); the carry (m0, E0, P0) at t0, updated to the chunk end on return. The sums of e^{s} use the chunk-end maximum M1 as a fixed
// reference (plain prefix sums); when the running maximum rises by more than e^60 inside the
// chunk, an exact (max, sum) scan is used instead so that nothing under- or overflows.
__device__ __forceinline__ void chunk_scan(Coef &cf, int lane, int t0, int nval, float sr_in, float g1v,
                                           float ghv, float s0, float &m0, float &E0, float &P0) {
    const int r = lane;
    const bool valid = r < nval;
    const float t0f = static_cast<float>(t0);
    const float sr = valid ? sr_in : 0.f;
    const float pp = wave_scan_add(sr);                             // sum of s over the chunk up to t
    const float mloc = wave_scan_max(valid ? sr : kNegInf);
    const float M = fmaxf(m0, mloc);                                 // m_t
    const float M1 = fmaxf(m0, lane_f(mloc, 63));                    // chunk-end maximum
    const float mfirst = lane_f(M, 0);
    // wave-uniform choice of the fixed-reference path
    const bool fixed_ref = __builtin_amdgcn_readfirstlane((M1 - mfirst <= 60.f) ? 1 : 0) != 0;
    float Et, dE, E0p;
    if (fixed_ref) {
        const float E0r = (m0 == kNegInf) ? 0.f : E0 * __expf(m0 - M1);
        const float pe = wave_scan_add(valid ? __expf(sr - M1) : 0.f);
        const float up = __expf(M1 - M);                             // 1 at the chunk end
        dE = pe * up;
        E0p = E0r * up;
        Et = E0p + dE;
    } else {
        float m = valid ? sr : kNegInf, e = valid ? 1.f : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float m2 = __shfl_up(m, off, 64);
            const float e2 = __shfl_up(e, off, 64);
            if (r >= off) lse_combine(m, e, m2, e2);
        }
        E0p = (m0 == kNegInf) ? 0.f : E0 * __expf(m0 - M);
        dE = (m == kNegInf) ? 0.f : e * __expf(m - M);
        Et = E0p + dE;
    }
    const float Pt = P0 + pp;
    const float s1 = __fdividef(1.f, 1.f + __expf(-g1v));
    const float sh = __fdividef(1.f, 1.f + __expf(-ghv));
    if (valid) {
        const float tt = t0f + static_cast<float>(r + 1);
        const float itt = __fdividef(1.f, tt);
        const float d1 = s1 - sh;
        const float a = __fdividef(sh, Et);
        // with the fixed reference, W uses e^{s_i - M1} e^{M1 - m_t}: fold the second factor in
        cf.qa[r] = fixed_ref ? a * __expf(M1 - M) : a;
        cf.qm[r] = M;
        cf.qb[r] = d1 * itt;
        // the zero-order term adds s0/t to gamma and so to the coefficient of H
        cf.qg[r] = -d1 * (Pt * itt) * itt + (s0 - sh) * itt;
        if (t0 > 0) {
            const float dt = tt - t0f;
            cf.qcx[r] = a * E0p;
            cf.qkap[r] = sh * __fdividef(E0p * dt - t0f * dE, Et * tt * t0f) +
                         d1 * __fdividef(P0 * dt - t0f * pp, tt * tt * t0f) + s0 * itt;
        } else {
            cf.qcx[r] = 0.f;
            cf.qkap[r] = 0.f;
        }
    }
    const int last = __builtin_amdgcn_readfirstlane(nval - 1);
    const float E1 = lane_f(Et, last), P1 = lane_f(Pt, last);
    const float dE1 = lane_f(dE, last), dP1 = lane_f(pp, last), E0p1 = lane_f(E0p, last);
    const float t1 = t0f + static_cast<float>(nval);
    const float iE1 = __fdividef(1.f, E1), it1 = __fdividef(1.f, t1);
    const float ek = valid ? __expf(sr - M1) : 0.f;
    cf.ek[r] = ek;
    cf.wx[r] = valid ? ek * iE1 - it1 : 0.f;
    cf.wy[r] = valid ? sr - P1 * it1 : 0.f;
    cf.s[r] = sr;
    if (r == 0) {
        cf.chunk[0] = M1;
        cf.chunk[1] = E1;
        cf.chunk[2] = P1;
        cf.chunk[6] = fixed_ref ? 0.f : 1.f;
        if (t0 > 0) {
            cf.chunk[3] = E0p1 * iE1;
            cf.chunk[4] = __fdividef(E0p1 * (t1 - t0f) - t0f * dE1, E1 * t0f * t1);
            cf.chunk[5] = __fdividef(P0 * (t1 - t0f) - t0f * dP1, t0f * t1);
        } else {
            cf.chunk[3] = cf.chunk[4] = cf.chunk[5] = 0.f;
        }
    }
    m0 = M1;
    E0 = E1;
    P0 = P1;
}



// ---- per-chunk coefficients ---------------------------------------------------------------
// One wave per (batch, head, chunk), all chunks in parallel: the logit carry at the chunk start
// (the given state's (m, E, P) merged with the aggregates of the earlier chunks) and the chunk's
// scalar scan. The record (sizeof(Coef) bytes) is read by the main scan pass. With scan segments the
// records are formed in the pass 1 launch (causal_seg_local_kernel), else by causal_coef_kernel.
constexpr int kCoefWaves = 4;
static_assert(sizeof(Coef) % 16 == 0, "coefficient records are copied in 16-byte pieces");
// LDS bytes of a coefficient record rounded up to whole 64-piece (1 KiB) wave copies
constexpr int kCoefLds = int((sizeof(Coef) / 16 + 63) / 64 * 64 * 16);
constexpr int kCoefStage = 8 * 64 * 16;   // one 64-piece direct copy per wave, up to 8 waves

// the record of chunk `item` (head item / nch, chunk item % nch), by one wave
__device__ __forceinline__ void coef_item(const Problem &p, const CausalWork &work, const int item, const int lane) {
    const int N = p.N;
    const int nch = (N + kC - 1) / kC;
    const int bh = item / nch, c = item % nch;
    const int t0 = c * kC, nval = min(kC, N - t0);
    const size_t row0 = static_cast<size_t>(bh) * N;
    const bool cont = p.sin.F != nullptr;
    const int tin = cont ? p.sin.t[bh] : 0;
    const bool from_state = cont && lane == 0;
    float m = from_state ? p.sin.m[bh] : kNegInf, e = from_state ? p.sin.E[bh] : 0.f;
    float ps = from_state ? p.sin.P[bh] : 0.f;
    const float4 *ag = work.agg + static_cast<size_t>(bh) * nch;
    for (int j = lane; j < c; j += 64) {
        const float4 a = ag[j];
        lse_combine(m, e, a.x, a.y);
        ps += a.z;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m, off, 64), e2 = __shfl_xor(e, off, 64), p2 = __shfl_xor(ps, off, 64);
        lse_combine(m, e, m2, e2);
        ps += p2;
    }
    float m0 = lane_f(m, 0), E0 = lane_f(e, 0), P0 = lane_f(ps, 0);
    const bool vs = lane < nval;
    const float sv = vs ? work.s[row0 + t0 + lane] : 0.f;
    const float g1v = vs ? lo_f(static_cast<const uint16_t *>(p.g1)[row0 + t0 + lane]) : 0.f;
    const float ghv = vs ? lo_f(static_cast<const uint16_t *>(p.gh)[row0 + t0 + lane]) : 0.f;
    const float s0 = (vs && p.g0 != nullptr)
                         ? __fdividef(1.f, 1.f + __expf(-lo_f(static_cast<const uint16_t *>(p.g0)[row0 + t0 + lane])))
                         : 0.f;
    chunk_scan(work.coef[item], lane, tin + t0, nval, sv, g1v, ghv, s0, m0, E0, P0);
}

__global__ __launch_bounds__(64 * kCoefWaves) void causal_coef_kernel(Problem p, CausalWork work) {
    const int nch = (p.N + kC - 1) / kC;
    const int item = blockIdx.x * kCoefWaves + (threadIdx.x >> 6);
    if (item >= p.B * p.H * nch) return;           // (wave-uniform)
    coef_item(p, work, item, threadIdx.x & 63);
}

// W piece of query block tb (0..3) and key-block pair pi (keys 32 pi .. 32 pi + 31), 2 pi <= tb:
// the six pieces the causal mask leaves non-zero.
__device__ __forceinline__ int w_piece(int tb, int pi) { return tb < 2 ? tb : 2 * tb - 2 + pi; }
__device__ __forceinline__ void piece_tb_pi(int piece, int &tb, int &pi) {
    tb = piece < 2 ? piece : (piece + 2) / 2;
    pi = piece < 2 ? 0 : piece & 1;
}

__device__ __forceinline__ void st16(unsigned char *p, const bf16x8 &v) { *reinterpret_cast<bf16x8 *>(p) = v; }
__device__ __forceinline__ bf16x8 ld16(const unsigned char *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// ---- segment-parallel scan ----------------------------------------------------------------
//
// The chunks of a head are cut into nseg segments of seg_chunks chunks. One workgroup of D/16 waves
// owns a whole head (wave w: value columns [16w, 16w+16), all D state rows of X, Y, H in float32
// registers) for one segment, so every chunk's q^, k^ and weights are formed once per head.
//
// Within a segment the per-chunk recurrence of the centred states is affine:
//   X <- rX X + cHX H + dX,   Y <- Y + cHY H + dY,   H <- H + dH        (d: the chunk's K^T V')
// so the state at the end of a segment is M (state at its start) + L, where L is the recurrence run
// from zero over the segment and M composes the scalar maps: X <- Rs X + Hs H, Y <- Y + Ys H.
//   pass 1 (PASS1 = true), segments 0 .. nseg-2: L and (Rs, Hs, Ys);
//   combine: start states of segments 1 .. nseg-1, in order, in float32;
//   main (PASS1 = false), every segment: from its start state, outputs of its chunks (and the final
//   recurrent state in the last segment).
// The float32 arithmetic is the sequential recurrence reassociated at segment boundaries.

// Segment states are stored in accumulator order: float4 index ((s * D/16 + jb) * D/16 + w) * 64 +
// lane holds rows 16 jb + 4 (lane >> 4) + i, i < 4, column 16 w + (lane & 15) of state s (X, Y, H).
template <int D> constexpr size_t kSegFloats = size_t(3) * D * D;

// one wave per 16 value columns: 8 waves (two per SIMD) at d = 128, 4 at d = 64
template <int D> constexpr int kScanThreads = 4 * D;

template <int D, bool ROPE, bool PASS1>
__global__ __launch_bounds__(kScanThreads<D>) void causal_scan_kernel(Problem p, CausalWork work) {
    constexpr int NW = D / 16;          // waves
    constexpr int NT = kScanThreads<D>;
    constexpr int CT = D / (16 * NW);   // 16-column tiles of the value dimension per wave
    constexpr int NGT = D / 16;         // 16-column tiles of a head (= 16-row state tiles)
    constexpr int KS = D / 32;          // 32-feature steps of the carried-state products
    constexpr int JB = D / 16;          // 16-row state tiles
    constexpr int TPR = NT / kC;        // prep threads per token row
    constexpr int FB = D / (16 * TPR);  // 16-feature blocks per prep thread
    constexpr int RP = kC * D / 8;      // 16-byte pieces of one chunk's rows of q (or k)
    static_assert(CT == 1 && FB >= 1, "d must be 64 or 128");
    // wave w's threads take rows [kC w / NW, kC (w + 1) / NW) in step 1, RP / NW pieces
    static_assert(kC % NW == 0 && (RP / NW) % 64 == 0 && RP / NW == (kC / NW) * (D / 8), "copy split");

    // Separate LDS objects, so that the compiler can tell the target of the direct global-to-LDS
    // copies (raw rows of the next chunk) from the buffers read meanwhile, and does not wait for
    // the copies before reading them.
    // raw bf16 rows of the next chunk, copied by direct global-to-LDS loads (16-byte pieces)
    __shared__ __align__(16) uint16_t s_rawk[kC * D];
    __shared__ __align__(16) uint16_t s_rawq[PASS1 ? 8 : kC * D];
    // unit, rotated rows of this chunk
    __shared__ __align__(16) uint16_t s_kh[kC][D + kPad];
    __shared__ __align__(16) uint16_t s_qh[PASS1 ? 1 : kC][D + kPad];
    // intra-chunk weights as B operands of V^T W^T, piece w_piece(tb, pi) x 64 lanes x 16 bytes
    __shared__ __align__(16) unsigned char s_wop[PASS1 ? 16 : 6 * 1024];
    // per wave: the v rows of its 16 value columns (64 tokens x 16 columns, token-major), copied by
    // direct global-to-LDS loads and read transposed in step 3
    __shared__ __align__(16) uint16_t s_rawv[NW][kC][kTile];
    // the coefficient record of the next chunk as it arrives by direct copy (s_cfS), and the current
    // chunk's (s_cfC), copied over from s_cfS at the start of the chunk: the copies always target
    // the one object, which is never read while they are in flight (a copy whose target is not a
    // fixed object makes the compiler wait for it before every later LDS access). A wave's direct
    // copy writes 64 pieces of 16 bytes: the buffers are padded to whole copies, so the lanes past
    // the record's end write into the padding. The RoPE phase of the chunk start (revolutions, in
    // [-1/2, 1/2]) is double-buffered: the next chunk's is written meanwhile.
    // one 64-piece copy per wave (D / 16 waves); a fixed size (with a size that depends on D the
    // host compiler drops the kernel's launch stub)
    __shared__ __align__(16) unsigned char s_cfS_raw[kCoefStage];
    static_assert(NW * 64 * 16 <= kCoefStage, "coefficient staging buffer");
    __shared__ __align__(16) unsigned char s_cfC_raw[kCoefLds];
    Coef &s_cfS = *reinterpret_cast<Coef *>(s_cfS_raw);
    const Coef &s_cfC = *reinterpret_cast<const Coef *>(s_cfC_raw);
    __shared__ float s_revA[D / 2];
    __shared__ float s_revB[D / 2];
    __shared__ float s_rpp[D / 2];       // RoPE revolutions per position of pair j
    __shared__ double s_rppd[D / 2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nseg = work.nseg;
    const int seg = blockIdx.x % (PASS1 ? nseg - 1 : nseg);
    const int bh = blockIdx.x / (PASS1 ? nseg - 1 : nseg);
    const int N = p.N;
    const int nch = (N + kC - 1) / kC;
    const int c_begin = seg * work.seg_chunks;
    const int c_end = min(nch, c_begin + work.seg_chunks);
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint16_t *qg = static_cast<const uint16_t *>(p.q) + row0 * D;
    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + row0 * D;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + row0 * D;
    uint16_t *og = static_cast<uint16_t *>(p.o) + row0 * D;
    // a sequence continued from a state: tokens are positions tin + 1 ..., and the first segment
    // of the main pass starts from that state
    const bool cont = p.sin.F != nullptr;
    const int tin = cont ? p.sin.t[bh] : 0;

    // state of this wave's column tiles gt = CT w + ct: X, Y, H rows 16 jb + 4 g4 + i, column
    // 16 gt + l16
    f32x4 X[CT][JB], Y[CT][JB], Hm[CT][JB];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int gt = CT * w + ct;
        const size_t sidx = static_cast<size_t>(gt) * 64 + lane;     // float4 index inside a (s, jb) block
        if (!PASS1 && seg == 0 && tin > 0) {
            // the given state in the centred basis: X = F/E - H/t, Y = G - (P/t) H
            const size_t mat0 = static_cast<size_t>(bh) * D * D;
            const float iE = 1.f / p.sin.E[bh], it = 1.f / static_cast<float>(tin);
            const float pt = p.sin.P[bh] * it;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t idx = mat0 + static_cast<size_t>(16 * jb + 4 * g4 + i) * D + gt * kTile + l16;
                    const float hh = p.sin.Hs[idx];
                    X[ct][jb][i] = p.sin.F[idx] * iE - hh * it;
                    Y[ct][jb][i] = p.sin.G[idx] - pt * hh;
                    Hm[ct][jb][i] = hh;
                }
        } else if (!PASS1 && seg > 0) {
            const float4 *st0 = reinterpret_cast<const float4 *>(work.segst + (static_cast<size_t>(bh) * (nseg - 1) + seg - 1) * kSegFloats<D>);
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                const float4 a = st0[(size_t(0 * JB + jb) * NGT) * 64 + sidx];
                const float4 b = st0[(size_t(1 * JB + jb) * NGT) * 64 + sidx];
                const float4 c = st0[(size_t(2 * JB + jb) * NGT) * 64 + sidx];
                X[ct][jb] = f32x4{a.x, a.y, a.z, a.w};
                Y[ct][jb] = f32x4{b.x, b.y, b.z, b.w};
                Hm[ct][jb] = f32x4{c.x, c.y, c.z, c.w};
            }
        } else {
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                for (int i = 0; i < 4; ++i) X[ct][jb][i] = Y[ct][jb][i] = Hm[ct][jb][i] = 0.f;
        }
    }
    // composed scalar map of the segment (pass 1): X <- Rs X + alp H + ..., Y <- Y + bet H + ...,
    // with Rs the exact product of the chunk factors rX
    float Rs = 1.f;
    // The X registers hold Z = X / rho. Per chunk the map X <- rX X + cHX H becomes rho <- rX rho and
    // Z += (cHX / rho) H, with the update operands scaled by 1/rho (Z += K^T diag(w_X / rho) V) and the
    // output coefficient of the X product by rho, so the multiply by rX disappears. The H couplings
    // of X and Y stay explicit: late in a sequence X and Y are far smaller than their H terms, and
    // carrying those terms as scalars too would make the states and update weights cancel before
    // bf16 rounding. rho is folded back into Z before it drops below 2^-40, and rX is floored at
    // 2^-40 (a change of at most 2^-40 |X| where the exact factor is smaller), so 1/rho stays within
    // 2^80. alp and bet are the composed H coefficients of X and Y (pass 1's segment map).
    float rho = 1.f, alp = 0.f, bet = 0.f;

    if (ROPE && tid < D / 2) {
        const double rev = rope_rev_per_pos(tid, D, p.rope_base);
        s_rpp[tid] = static_cast<float>(rev);
        s_rppd[tid] = rev;
        double r = static_cast<double>(tin + c_begin * kC) * rev;
        s_revA[tid] = static_cast<float>(r - rint(r));
    }

    // the v rows of this wave's columns 16 w + [0, 16) of chunk c into s_rawv[w] by direct copies:
    // 128 pieces of 16 bytes, piece p = (token p >> 1, half p & 1), rows past N read row N - 1
    // (finite; every product they enter is zero: the k^ rows and W columns of absent tokens are
    // zero). Each wave copies exactly the tile it reads, after its own last read of the previous one.
    auto fetch_vt = [&](const int c) __attribute__((always_inline)) {
        static_assert(CT == 1 && kC * kTile * 2 == 2 * 64 * 16, "v tile: two 64-piece copies per wave");
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pc = 64 * i + lane;
            const int t_ = min(c * kC + (pc >> 1), N - 1);
            const uint4 *src = reinterpret_cast<const uint4 *>(vg + static_cast<size_t>(t_) * D + w * kTile + 8 * (pc & 1));
            __builtin_amdgcn_global_load_lds(src, reinterpret_cast<unsigned char *>(&s_rawv[w][0][0]) + i * 1024, 16, 0, 0);
        }
    };
    // the coefficient record and the raw q and k rows of chunk c into LDS: the chunk's rows are
    // contiguous in memory, so piece i (16 bytes) is element 8 i of the block; pieces past the
    // last token repeat the last valid piece (the rows they fill are zeroed when read). Wave w
    // copies exactly the pieces its own threads read next: rows [kC w / NW, kC (w + 1) / NW) of q
    // and k in step 1, and pieces [64 w, 64 w + 64) of the record in the copy to s_cfC, so each
    // wave's wait for its own copies (which the compiler places) is all the reads need.
    auto fetch_raw = [&](const int c) __attribute__((always_inline)) {
        {
            // every wave issues one copy (the waves past the record copy its last piece into their
            // part of the padding): the same memory operations on every wave and trip, so the
            // waits the compiler places for them are exact counts
            constexpr int CP = int(sizeof(Coef) / 16);
            static_assert(CP <= NT, "the record fits one copy per wave");
            const uint4 *srcc = reinterpret_cast<const uint4 *>(work.coef + static_cast<size_t>(bh) * nch + c);
            __builtin_amdgcn_global_load_lds(srcc + min(w * 64 + lane, CP - 1), s_cfS_raw + w * 64 * 16, 16, 0, 0);
        }
        const int nv = min(kC, N - c * kC) * (D / 8);
        const uint4 *srck = reinterpret_cast<const uint4 *>(kg + static_cast<size_t>(c) * kC * D);
        const uint4 *srcq = reinterpret_cast<const uint4 *>(qg + static_cast<size_t>(c) * kC * D);
#pragma unroll
        for (int i = 0; i < RP / NT; ++i) {
            const int base = w * (RP / NW) + i * 64;             // wave-uniform
            __builtin_amdgcn_global_load_lds(srck + min(base + lane, nv - 1),
                                             reinterpret_cast<unsigned char *>(s_rawk) + base * 16, 16, 0, 0);
            if (!PASS1)
                __builtin_amdgcn_global_load_lds(srcq + min(base + lane, nv - 1),
                                                 reinterpret_cast<unsigned char *>(s_rawq) + base * 16, 16, 0, 0);
        }
    };
    if (c_begin < c_end) {
        fetch_raw(c_begin);
        fetch_vt(c_begin);
    }
    // unconditional: the start-state loads and the first copies are complete on every path into
    // the loop
    __syncthreads();

    // the k^T operand of row tile jb (features 16 jb + l16) and key step ks2, in kperm order (keys
    // 32 ks2 + 4 g4 + [0, 4), then + 16), straight from the k^ rows by two transposing reads: lane
    // (g4, l16) names features 16 jb + 4 (l16 & 3) + [0, 4) of key 32 ks2 + 4 g4 + (l16 >> 2)
    auto k_operand = [&](const int jb, const int ks2) __attribute__((always_inline)) {
        const int f = 16 * jb + 4 * (l16 & 3);
        const int r0 = 32 * ks2 + 4 * g4 + (l16 >> 2);
        const uint2 a = lds_tr16(&s_kh[r0][f]);
        const uint2 b = lds_tr16(&s_kh[r0 + 16][f]);
        return as_bf16x8(a.x, a.y, b.x, b.y);
    };

    // one chunk: its start phase in revc, the next chunk's written into revn
    auto chunk = [&](const int c, const float *revc, float *revn) __attribute__((always_inline)) {
        const int t0 = c * kC;
        const int nval = min(kC, N - t0);
        const bool has_prev = tin + t0 > 0;      // tokens before this chunk (a carried state)
        // this chunk's coefficient record, from the copy's target to the buffer read below (published
        // by the barrier after step 1)
        if (tid < int(sizeof(Coef) / 16))
            reinterpret_cast<uint4 *>(s_cfC_raw)[tid] = reinterpret_cast<const uint4 *>(s_cfS_raw)[tid];

        // ---- (1) unit, rotated q^ and k^ rows: thread = (row r, FB blocks of 16 features)
        {
            const int r = tid / TPR;
            const bool valid = r < nval;
            uint4 k4[FB][2], q4[FB][2];
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int f0 = 16 * ((tid % TPR) * FB + fb) + 8 * h;
                    k4[fb][h] = valid ? *reinterpret_cast<const uint4 *>(&s_rawk[r * D + f0]) : make_uint4(0, 0, 0, 0);
                    if (!PASS1)
                        q4[fb][h] = valid ? *reinterpret_cast<const uint4 *>(&s_rawq[r * D + f0]) : make_uint4(0, 0, 0, 0);
                }
            float ssk = 0.f, ssq = 0.f;
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    ssk = dot2_bf16(k4[fb][h].x, ssk); ssk = dot2_bf16(k4[fb][h].y, ssk);
                    ssk = dot2_bf16(k4[fb][h].z, ssk); ssk = dot2_bf16(k4[fb][h].w, ssk);
                    if (!PASS1) {
                        ssq = dot2_bf16(q4[fb][h].x, ssq); ssq = dot2_bf16(q4[fb][h].y, ssq);
                        ssq = dot2_bf16(q4[fb][h].z, ssq); ssq = dot2_bf16(q4[fb][h].w, ssq);
                    }
                }
            ssk = group_sum<TPR>(ssk);
            const float ik = valid ? __frsqrt_rn(fmaxf(ssk, 1e-24f)) : 0.f;
            float iq = 0.f;
            if (!PASS1) {
                ssq = group_sum<TPR>(ssq);
                iq = valid ? __frsqrt_rn(fmaxf(ssq, 1e-24f)) : 0.f;
            }
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int blk = 2 * ((tid % TPR) * FB + fb) + h;     // 8-feature block
                    uint32_t wk[4] = {k4[fb][h].x, k4[fb][h].y, k4[fb][h].z, k4[fb][h].w};
                    uint32_t wq[4] = {q4[fb][h].x, q4[fb][h].y, q4[fb][h].z, q4[fb][h].w};
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        float cs = 1.f, sn = 0.f;
                        if (ROPE) {
                            // phase of position tin + t0 + r for pair j, in revolutions
                            const int j = 4 * blk + b;
                            float rev = fmaf(static_cast<float>(r), s_rpp[j], revc[j]);
                            rev -= rintf(rev);
                            cs = __builtin_amdgcn_cosf(rev);
                            sn = __builtin_amdgcn_sinf(rev);
                        }
                        const float k0 = lo_f(wk[b]), k1 = hi_f(wk[b]);
                        const float ck = cs * ik, sk = sn * ik;
                        wk[b] = pack2(k0 * ck - k1 * sk, k0 * sk + k1 * ck);
                        if (!PASS1) {
                            const float q0 = lo_f(wq[b]), q1 = hi_f(wq[b]);
                            const float cq = cs * iq, sq = sn * iq;
                            wq[b] = pack2(q0 * cq - q1 * sq, q0 * sq + q1 * cq);
                        }
                    }
                    *reinterpret_cast<uint4 *>(&s_kh[r][8 * blk]) = make_uint4(wk[0], wk[1], wk[2], wk[3]);
                    if (!PASS1) *reinterpret_cast<uint4 *>(&s_qh[r][8 * blk]) = make_uint4(wq[0], wq[1], wq[2], wq[3]);
                }
            if (ROPE && tid < D / 2 && c + 1 < c_end) {
                const double r2 = static_cast<double>(tin + t0 + kC) * s_rppd[tid];
                revn[tid] = static_cast<float>(r2 - rint(r2));
            }
        }
        lds_barrier();

        // ---- (2) next chunk's record and raw rows in flight; A^T and W
        // unconditional (the last chunk fetches itself again, into buffers no longer read), so that
        // every trip issues the same memory operations and the waits for them are exact counts
        fetch_raw(min(c + 1, c_end - 1));
        if (!PASS1) {
            // the ten (query block tb, key block kb <= tb) tiles of A^T, spread over the waves; each
            // fills its half (8 bytes per lane) of the W piece of key pair kb / 2, and the tiles
            // (0, 0) and (2, 2) also the zero half whose keys all follow the queries
            const Coef &cf = s_cfC;
            const bool exact_exp = cf.chunk[6] != 0.f;
            for (int blk = w; blk < 10; blk += NW) {
                const int tb = blk < 1 ? 0 : blk < 3 ? 1 : blk < 6 ? 2 : 3;
                const int kb = blk - tb * (tb + 1) / 2;
                const int tq = 16 * tb + l16;
                const int key = 16 * kb + l16;
                f32x4 at = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 qop = *reinterpret_cast<const bf16x8 *>(&s_qh[tq][32 * ks + 8 * g4]);
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&s_kh[key][32 * ks + 8 * g4]);
                    at = mfma(a, qop, at);
                }
                const float qa = cf.qa[tq], qm = cf.qm[tq], qb = cf.qb[tq], qgm = cf.qg[tq];
                const float4 s4 = *reinterpret_cast<const float4 *>(&cf.s[16 * kb + 4 * g4]);
                const float ks_[4] = {s4.x, s4.y, s4.z, s4.w};
                float ke_[4];
                if (exact_exp) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) ke_[i] = __expf(ks_[i] - qm);
                } else {
                    const float4 e4 = *reinterpret_cast<const float4 *>(&cf.ek[16 * kb + 4 * g4]);
                    ke_[0] = e4.x; ke_[1] = e4.y; ke_[2] = e4.z; ke_[3] = e4.w;
                }
                float wt[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kk = 16 * kb + 4 * g4 + i;
                    const float x = at[i] * (qa * ke_[i] + qb * ks_[i] + qgm);
                    wt[i] = (kk <= tq && tq < nval) ? x : 0.f;
                }
                unsigned char *dst = s_wop + (size_t(w_piece(tb, kb >> 1)) * 64 + lane) * 16;
                *reinterpret_cast<uint2 *>(dst + (kb & 1) * 8) = make_uint2(pack2(wt[0], wt[1]), pack2(wt[2], wt[3]));
                if ((kb & 1) == 0 && kb + 1 > tb) *reinterpret_cast<uint2 *>(dst + 8) = make_uint2(0u, 0u);
            }
            lds_barrier();          // W is in LDS (pass 1 writes nothing in step 2)
        }

        // ---- (3) per wave: the carried-state products, V^T W^T, outputs, and the state update
        const Coef &cf = s_cfC;
        const float4 ch = make_float4(cf.chunk[3], cf.chunk[4], cf.chunk[5], cf.chunk[0]);   // rX, cHX, cHY, m1
        if (has_prev && rho < 0x1p-40f) {        // fold rho into Z (rare; the same on every lane)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) X[ct][jb][i] *= rho;
            rho = 1.f;
        }
        // scalars of the basis after this chunk (the first chunk of the sequence starts from nothing
        // and keeps them)
        const float rho1 = has_prev ? rho * fmaxf(ch.x, 0x1p-40f) : rho;
        const float alp1 = has_prev ? ch.x * alp + ch.y : alp;
        const float bet1 = has_prev ? bet + ch.z : bet;
        const float irho1 = 1.f / rho1;
        const float hz = has_prev ? ch.y * irho1 : 0.f;   // Z += hz H
        const float hy = has_prev ? ch.z : 0.f;           // Y += hy H

        // the v operands of this wave's column tile, in kperm order (keys 32 ks2 + 4 g4 + [0, 4), then
        // + 16), read transposed from its v rows (lane (g4, l16) names columns 4 (l16 & 3) + [0, 4) of
        // key 32 ks2 + 4 g4 + (l16 >> 2)): v itself (the H update and V^T W^T), and the update
        // operands v w_X / rho1, v w_Y with the keys' weights from the coefficient record
        // The wave's copies of this v tile (issued at the end of the previous chunk) are older than
        // the record and row copies of the next chunk issued in step 2 (kNewer of them). The
        // transposing reads carry no memory operand the compiler can match against the copies, so
        // it does not reliably wait for them: the wait is explicit.
        {
            constexpr int kNewer = 1 + RP / NT + (PASS1 ? 0 : RP / NT);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kNewer) : "memory");
        }
        bf16x8 BX[CT][kC / 32], BY[CT][kC / 32], BH[CT][kC / 32];
#pragma unroll
        for (int ks2 = 0; ks2 < kC / 32; ++ks2) {
            const int k0 = 32 * ks2 + 4 * g4;
            const int tok = k0 + (l16 >> 2);
            const uint2 va = lds_tr16(&s_rawv[w][tok][4 * (l16 & 3)]);
            const uint2 vb = lds_tr16(&s_rawv[w][tok + 16][4 * (l16 & 3)]);
            BH[0][ks2] = as_bf16x8(va.x, va.y, vb.x, vb.y);
            const float4 xa = *reinterpret_cast<const float4 *>(&cf.wx[k0]);
            const float4 xb = *reinterpret_cast<const float4 *>(&cf.wx[k0 + 16]);
            const float4 ya = *reinterpret_cast<const float4 *>(&cf.wy[k0]);
            const float4 yb = *reinterpret_cast<const float4 *>(&cf.wy[k0 + 16]);
            const float vv[8] = {lo_f(va.x), hi_f(va.x), lo_f(va.y), hi_f(va.y), lo_f(vb.x), hi_f(vb.x), lo_f(vb.y), hi_f(vb.y)};
            const float wxs[8] = {xa.x * irho1, xa.y * irho1, xa.z * irho1, xa.w * irho1,
                                  xb.x * irho1, xb.y * irho1, xb.z * irho1, xb.w * irho1};
            const float wys[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
            BX[0][ks2] = as_bf16x8(pack2(vv[0] * wxs[0], vv[1] * wxs[1]), pack2(vv[2] * wxs[2], vv[3] * wxs[3]),
                                   pack2(vv[4] * wxs[4], vv[5] * wxs[5]), pack2(vv[6] * wxs[6], vv[7] * wxs[7]));
            BY[0][ks2] = as_bf16x8(pack2(vv[0] * wys[0], vv[1] * wys[1]), pack2(vv[2] * wys[2], vv[3] * wys[3]),
                                   pack2(vv[4] * wys[4], vv[5] * wys[5]), pack2(vv[6] * wys[6], vv[7] * wys[7]));
        }

        // carried-state products and the state update, interleaved by pairs of row tiles: step ks
        // reads rows 2ks, 2ks+1 of Z, Y', H (as bf16 MFMA operands, the state at t0), after which
        // those rows are advanced by K^T V' on MFMA; each q^ and k^T operand serves every column
        // tile of the wave
        f32x4 ax[CT][4], ay[CT][4], ah[CT][4];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) ax[ct][tb][i] = ay[ct][tb][i] = ah[ct][tb][i] = 0.f;
        const bool carried = !PASS1 && has_prev;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (carried) {
                bf16x8 AX[CT], AY[CT], AH[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const f32x4 &x0 = X[ct][2 * ks], &x1 = X[ct][2 * ks + 1];
                    const f32x4 &y0 = Y[ct][2 * ks], &y1 = Y[ct][2 * ks + 1];
                    const f32x4 &h0 = Hm[ct][2 * ks], &h1 = Hm[ct][2 * ks + 1];
                    AX[ct] = as_bf16x8(pack2(x0[0], x0[1]), pack2(x0[2], x0[3]), pack2(x1[0], x1[1]), pack2(x1[2], x1[3]));
                    AY[ct] = as_bf16x8(pack2(y0[0], y0[1]), pack2(y0[2], y0[3]), pack2(y1[0], y1[1]), pack2(y1[2], y1[3]));
                    AH[ct] = as_bf16x8(pack2(h0[0], h0[1]), pack2(h0[2], h0[3]), pack2(h1[0], h1[1]), pack2(h1[2], h1[3]));
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    // q^ features {32 ks + 4 g4 + i, 32 ks + 16 + 4 g4 + i}: the order in which a lane
                    // holds the rows of the two 16-row state tiles
                    const uint2 qa = *reinterpret_cast<const uint2 *>(&s_qh[16 * tb + l16][32 * ks + 4 * g4]);
                    const uint2 qc = *reinterpret_cast<const uint2 *>(&s_qh[16 * tb + l16][32 * ks + 16 + 4 * g4]);
                    const bf16x8 Bq = as_bf16x8(qa.x, qa.y, qc.x, qc.y);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        ax[ct][tb] = mfma(AX[ct], Bq, ax[ct][tb]);
                        ay[ct][tb] = mfma(AY[ct], Bq, ay[ct][tb]);
                        ah[ct][tb] = mfma(AH[ct], Bq, ah[ct][tb]);
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int jb = 2 * ks + jj;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        X[ct][jb][i] += hz * Hm[ct][jb][i];
                        Y[ct][jb][i] += hy * Hm[ct][jb][i];
                    }
#pragma unroll
                for (int ks2 = 0; ks2 < kC / 32; ++ks2) {
                    const bf16x8 Ak = k_operand(jb, ks2);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        X[ct][jb] = mfma(Ak, BX[ct][ks2], X[ct][jb]);
                        Y[ct][jb] = mfma(Ak, BY[ct][ks2], Y[ct][jb]);
                        Hm[ct][jb] = mfma(Ak, BH[ct][ks2], Hm[ct][jb]);
                    }
                }
            }
        }
        if (PASS1) {
            // the first chunk of the sequence starts from nothing
            Rs = has_prev ? ch.x * Rs : 0.f;
        } else {
            // outputs: coefficients on the carried-state products, plus V^T W^T (intra-chunk)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int tq = 16 * tb + l16;
                // X = rho Z at t0 (without a carried state the products are zero and the
                // coefficients finite)
                const float cz = cf.qcx[tq] * rho, cb = cf.qb[tq], chh = cf.qkap[tq];
                // rows past the end go to a sink in the workspace: the store is unconditional
                uint16_t *dst = tq < nval ? og + static_cast<size_t>(t0 + tq) * D : work.sink + static_cast<size_t>(tq) * D;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    f32x4 oacc;
#pragma unroll
                    for (int i = 0; i < 4; ++i) oacc[i] = cz * ax[ct][tb][i] + cb * ay[ct][tb][i] + chh * ah[ct][tb][i];
#pragma unroll
                    for (int pi = 0; pi < 2; ++pi) {
                        if (2 * pi > tb) continue;
                        // V^T: keys {32 pi + 4 g4 + [0, 4)} and {32 pi + 16 + 4 g4 + [0, 4)}, which is
                        // BH (kperm order); the second half is zero where all its keys follow the queries
                        bf16x8 vt = BH[ct][pi];
                        if (2 * pi + 1 > tb) vt[4] = vt[5] = vt[6] = vt[7] = 0;
                        const bf16x8 Bw = ld16(s_wop + (size_t(w_piece(tb, pi)) * 64 + lane) * 16);
                        oacc = mfma(vt, Bw, oacc);
                    }
                    const uint2 ov = make_uint2(pack2(oacc[0], oacc[1]), pack2(oacc[2], oacc[3]));
                    *reinterpret_cast<uint2 *>(dst + (CT * w + ct) * kTile + 4 * g4) = ov;
                }
            }
        }
        rho = rho1;
        alp = alp1;
        bet = bet1;
        // next chunk's v tile, after this wave's reads of this one (their values are in use above)
        fetch_vt(min(c + 1, c_end - 1));
        // LDS reads and writes of this chunk done everywhere. No memory fence: it would wait for the
        // copies just issued; the direct copies of chunk c + 1 are read only by the wave that issued
        // them, after the wait the compiler places for it.
        lds_barrier();
    };
    for (int c = c_begin; c < c_end; ++c) {
        const bool odd = ((c - c_begin) & 1) != 0;      // the segment's chunks alternate phase buffers
        chunk(c, odd ? s_revB : s_revA, odd ? s_revA : s_revB);
    }

    // back to the plain basis: X = rho Z
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int i = 0; i < 4; ++i) X[ct][jb][i] *= rho;
    if (PASS1) {
        // segment-local sums and the composed scalar map, for the combine step
        float4 *dst = reinterpret_cast<float4 *>(work.segst + (static_cast<size_t>(bh) * (nseg - 1) + seg) * kSegFloats<D>);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const size_t sidx = static_cast<size_t>(CT * w + ct) * 64 + lane;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                dst[(size_t(0 * JB + jb) * NGT) * 64 + sidx] = make_float4(X[ct][jb][0], X[ct][jb][1], X[ct][jb][2], X[ct][jb][3]);
                dst[(size_t(1 * JB + jb) * NGT) * 64 + sidx] = make_float4(Y[ct][jb][0], Y[ct][jb][1], Y[ct][jb][2], Y[ct][jb][3]);
                dst[(size_t(2 * JB + jb) * NGT) * 64 + sidx] = make_float4(Hm[ct][jb][0], Hm[ct][jb][1], Hm[ct][jb][2], Hm[ct][jb][3]);
            }
        }
        if (tid == 0) work.segsc[static_cast<size_t>(bh) * nseg + seg] = make_float4(Rs, alp, bet, 0.f);
        return;
    }

    // ---- final recurrent state (last segment): back to F = E (X + H/t), G = Y + (P/t) H
    if (p.st.F != nullptr && seg == nseg - 1) {
        // the logit carry after the last chunk: its coefficient record, still in s_cfC
        const Coef &cl = s_cfC;
        const float mE = cl.chunk[0], EE = cl.chunk[1], PE = cl.chunk[2];
        const size_t mat0 = static_cast<size_t>(bh) * D * D;
        const float tf = static_cast<float>(tin + N);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float hh = Hm[ct][jb][i];
                    const int j = 16 * jb + 4 * g4 + i;
                    const size_t idx = mat0 + static_cast<size_t>(j) * D + (CT * w + ct) * kTile + l16;
                    p.st.F[idx] = N > 0 ? EE * (X[ct][jb][i] + hh / tf) : 0.f;
                    p.st.G[idx] = N > 0 ? Y[ct][jb][i] + (PE / tf) * hh : 0.f;
                    p.st.Hs[idx] = hh;
                }
        const int nls = (N + kLogitSeg - 1) / kLogitSeg;
        for (int f = tid; f < D; f += NT) {
            float su = cont ? p.sin.Su[static_cast<size_t>(bh) * D + f] : 0.f;
            for (int sg = 0; sg < nls; ++sg) su += work.useg[(static_cast<size_t>(bh) * nls + sg) * D + f];
            p.st.Su[static_cast<size_t>(bh) * D + f] = su;
        }
        if (tid == 0) {
            p.st.m[bh] = N > 0 ? mE : kNegInf;
            p.st.E[bh] = N > 0 ? EE : 0.f;
            p.st.P[bh] = N > 0 ? PE : 0.f;
            p.st.t[bh] = tin + N;
        }
    }
}

// ---- pass 1, token-parallel: the segment-local state L of segments 0 .. nseg-2 (the recurrence run
// from zero over the segment) in the centred basis at the segment end. Unrolled, the chunk maps
// X <- rX X + cHX H + dX, Y <- Y + cHY H + dY, H <- H + dH of a segment give per token i
//   L_X = sum_i (e^{s_i - m_n}/E_n - 1/t_n) k^_i^T v_i,   L_Y = sum_i (s_i - P_n/t_n) k^_i^T v_i,
//   L_H = sum_i k^_i^T v_i,
// with (m_n, E_n, P_n) the logit carry and t_n the token count at the segment end (the centred
// weights of 关键设计 at t_n): one weighted contraction over the segment's tokens (kv_states.hpp),
// with no chain of per-chunk steps. The segment's map of its start state (X <- Rs X + Hs H,
// Y <- Y + Ys H) is the same re-centring between the carries at its two ends:
//   Rs = E_s e^{m_s - m_n} / E_n,   Hs = Rs / t_s - 1 / t_n,   Ys = P_s / t_s - P_n / t_n.
// Both carries come from the per-chunk logit aggregates, so pass 1 does not wait for the chunk
// records: the same launch also forms them, in the workgroups past the segments (one wave per
// chunk), which take the CUs the segments leave free.
template <int D, bool ROPE>
__global__ __launch_bounds__(kv_threads<D>()) void causal_seg_local_kernel(Problem p, CausalWork work) {
    constexpr int JB = D / 16, NGT = D / 16;
    __shared__ __align__(16) KvSmem<D, 3> sm;
    __shared__ double rev[ROPE ? D / 2 : 1];
    __shared__ float scal[3];
    const int nseg = work.nseg;
    const int N = p.N, nch = (N + kC - 1) / kC;
    const int nloc = p.B * p.H * (nseg - 1);
    if (static_cast<int>(blockIdx.x) >= nloc) {
        // coefficient records (whole workgroup: no barrier below is reached)
        const int item = (static_cast<int>(blockIdx.x) - nloc) * (kv_threads<D>() / 64) + static_cast<int>(threadIdx.x >> 6);
        if (item < p.B * p.H * nch) coef_item(p, work, item, threadIdx.x & 63);
        return;
    }
    const int seg = blockIdx.x % (nseg - 1), bh = blockIdx.x / (nseg - 1);
    const int c_begin = seg * work.seg_chunks, c_end = min(nch, c_begin + work.seg_chunks);
    const int t0 = c_begin * kC, t1 = min(N, c_end * kC);
    const bool cont = p.sin.F != nullptr;
    const int tin = cont ? p.sin.t[bh] : 0;
    const size_t row0 = static_cast<size_t>(bh) * N;
    // tokens of this call are positions tin + r (RoPE phase as in the main pass)
    KvStates<D, ROPE, 3> kv(sm, static_cast<const uint16_t *>(p.k) + row0 * D, static_cast<const uint16_t *>(p.v) + row0 * D,
                            work.s + row0, rev, N, t0, t1, tin);
    kv.start();
    if (ROPE && kv.tid < D / 2) rev[kv.tid] = rope_rev_per_pos(kv.tid, D, p.rope_base);
    if (kv.wv == 0) {
        // carries at the segment start (chunks before c_begin) and end (before c_end), from the given
        // state's (m, E, P) and the chunk aggregates
        const bool from_state = cont && kv.lane == 0;
        float ms = from_state ? p.sin.m[bh] : kNegInf, es = from_state ? p.sin.E[bh] : 0.f, ps = from_state ? p.sin.P[bh] : 0.f;
        float me = kNegInf, ee = 0.f, pe = 0.f;
        const float4 *ag = work.agg + static_cast<size_t>(bh) * nch;
        for (int j = kv.lane; j < c_end; j += 64) {
            const float4 g = ag[j];
            if (j < c_begin) {
                lse_combine(ms, es, g.x, g.y);
                ps += g.z;
            } else {
                lse_combine(me, ee, g.x, g.y);
                pe += g.z;
            }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            float m2 = __shfl_xor(ms, off, 64), e2 = __shfl_xor(es, off, 64), p2 = __shfl_xor(ps, off, 64);
            lse_combine(ms, es, m2, e2);
            ps += p2;
            m2 = __shfl_xor(me, off, 64), e2 = __shfl_xor(ee, off, 64), p2 = __shfl_xor(pe, off, 64);
            lse_combine(me, ee, m2, e2);
            pe += p2;
        }
        // end carry = start carry merged with the segment's own chunks
        float mn = ms, en = es;
        lse_combine(mn, en, me, ee);
        const float pn = ps + pe;
        if (kv.lane == 0) {
            scal[0] = mn;
            scal[1] = en;
            scal[2] = pn;
            const float ts = static_cast<float>(tin + t0), tn = static_cast<float>(tin + t1);
            float Rs = 0.f, hs = 0.f, ys = 0.f;          // from nothing: the start state is zero
            if (tin + t0 > 0) {
                Rs = es * __expf(ms - mn) / en;
                hs = Rs / ts - 1.f / tn;
                ys = ps / ts - pn / tn;
            }
            work.segsc[static_cast<size_t>(bh) * nseg + seg] = make_float4(Rs, hs, ys, 0.f);
        }
    }
    lds_barrier();
    const float mn = scal[0], iE = 1.f / scal[1], itn = 1.f / static_cast<float>(tin + t1), pn = scal[2] * itn;
    kv.run([&](float sv) __attribute__((always_inline)) { return make_float2(__expf(sv - mn) * iE - itn, sv - pn); });
    // the segment state layout: float4 ((s JB + jb) NGT + gt) 64 + lane holds rows 16 jb + 4 g4 + [0, 4)
    // of column 16 gt + l16 of state s
    float4 *dst = reinterpret_cast<float4 *>(work.segst + (static_cast<size_t>(bh) * (nseg - 1) + seg) * kSegFloats<D>);
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
            dst[(size_t(s * JB + jb) * NGT + kv.wv) * 64 + kv.lane] =
                make_float4(kv.acc[s][jb][0], kv.acc[s][jb][1], kv.acc[s][jb][2], kv.acc[s][jb][3]);
}

// Start states of segments 1 .. nseg-1 (in place over the segment-local sums), one float4 position
// of the three state matrices per thread: S_{j+1} = M_j S_j + L_j with S_0 = 0, or the given state
// in the centred basis for a continued sequence.
template <int D>
__global__ __launch_bounds__(256) void causal_seg_combine_kernel(Problem p, CausalWork work) {
    constexpr size_t Q = size_t(D) * D / 4;              // float4 positions per state matrix
    constexpr int kMaxSeg = 8;                           // segment-local sums loaded up front
    const size_t pos = static_cast<size_t>(blockIdx.y) * 256 + threadIdx.x;
    if (pos >= Q) return;
    const int bh = blockIdx.x;
    const int nseg = work.nseg;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x, h = x;
    const int tin = p.sin.F != nullptr ? p.sin.t[bh] : 0;
    if (tin > 0) {
        // float4 position pos of a segment state holds rows 16 jb + 4 g4 + [0, 4) of column
        // 16 w + l16, with pos = (jb (d/16) + w) 64 + 16 g4 + l16 (the scan kernel's register order)
        constexpr int NW = D / 16;
        const int jb = static_cast<int>(pos / (NW * 64)), rem = static_cast<int>(pos % (NW * 64));
        const int col = 16 * (rem / 64) + (rem & 15), row = 16 * jb + 4 * ((rem & 63) >> 4);
        const size_t base = static_cast<size_t>(bh) * D * D + static_cast<size_t>(row) * D + col;
        const float iE = 1.f / p.sin.E[bh], it = 1.f / static_cast<float>(tin);
        const float pt = p.sin.P[bh] * it;
        float xs[4], ys[4], hs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            hs[i] = p.sin.Hs[base + static_cast<size_t>(i) * D];
            xs[i] = p.sin.F[base + static_cast<size_t>(i) * D] * iE - hs[i] * it;
            ys[i] = p.sin.G[base + static_cast<size_t>(i) * D] - pt * hs[i];
        }
        x = make_float4(xs[0], xs[1], xs[2], xs[3]);
        y = make_float4(ys[0], ys[1], ys[2], ys[3]);
        h = make_float4(hs[0], hs[1], hs[2], hs[3]);
    }
    for (int j0 = 0; j0 + 1 < nseg; j0 += kMaxSeg) {
        const int nj = min(kMaxSeg, nseg - 1 - j0);
        float4 lx[kMaxSeg], ly[kMaxSeg], lh[kMaxSeg];
#pragma unroll
        for (int jj = 0; jj < kMaxSeg; ++jj) {
            if (jj < nj) {
                const float4 *st = reinterpret_cast<const float4 *>(work.segst + (static_cast<size_t>(bh) * (nseg - 1) + j0 + jj) * kSegFloats<D>);
                lx[jj] = st[pos];
                ly[jj] = st[Q + pos];
                lh[jj] = st[2 * Q + pos];
            }
        }
#pragma unroll
        for (int jj = 0; jj < kMaxSeg; ++jj) {
            if (jj < nj) {
                float4 *st = reinterpret_cast<float4 *>(work.segst + (static_cast<size_t>(bh) * (nseg - 1) + j0 + jj) * kSegFloats<D>);
                const float4 m = work.segsc[static_cast<size_t>(bh) * nseg + j0 + jj];   // Rs, Hs, Ys
                const float4 nx = make_float4(m.x * x.x + m.y * h.x + lx[jj].x, m.x * x.y + m.y * h.y + lx[jj].y,
                                              m.x * x.z + m.y * h.z + lx[jj].z, m.x * x.w + m.y * h.w + lx[jj].w);
                const float4 ny = make_float4(y.x + m.z * h.x + ly[jj].x, y.y + m.z * h.y + ly[jj].y,
                                              y.z + m.z * h.z + ly[jj].z, y.w + m.z * h.w + ly[jj].w);
                const float4 nh = make_float4(h.x + lh[jj].x, h.y + lh[jj].y, h.z + lh[jj].z, h.w + lh[jj].w);
                st[pos] = nx;
                st[Q + pos] = ny;
                st[2 * Q + pos] = nh;
                x = nx;
                y = ny;
                h = nh;
            }
        }
    }
}


template <int D, bool ROPE>
hipError_t launch_one(const Problem &p, const CausalWork &w, hipStream_t stream) {
    hipError_t err;
    const int bh = p.B * p.H;
    const int nch = (p.N + kC - 1) / kC;
    if (w.nseg > 1) {
        // pass 1, and the coefficient records in the workgroups past the segments
        constexpr int kWaves = kv_threads<D>() / 64;
        const int ncoef = (bh * nch + kWaves - 1) / kWaves;
        hipLaunchKernelGGL((causal_seg_local_kernel<D, ROPE>), dim3(bh * (w.nseg - 1) + ncoef), dim3(kv_threads<D>()), 0,
                           stream, p, w);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL((causal_seg_combine_kernel<D>), dim3(bh, (D * D / 4 + 255) / 256), dim3(256), 0,
                           stream, p, w);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    } else if (nch > 0) {
        hipLaunchKernelGGL(causal_coef_kernel, dim3((bh * nch + kCoefWaves - 1) / kCoefWaves), dim3(64 * kCoefWaves), 0,
                           stream, p, w);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    hipLaunchKernelGGL((causal_scan_kernel<D, ROPE, false>), dim3(bh * w.nseg), dim3(kScanThreads<D>),
                       0, stream, p, w);
    return hipGetLastError();
}

}  // namespace

// Segments of the scan: enough (head, segment) workgroups to cover the chip, whole chunks each.
static void seg_plan(int B, int H, int N, int &nseg, int &seg_chunks) {
    const int nch = (N + kC - 1) / kC;
    const int bh = B * H;
    int want = (256 + bh - 1) / bh;
    if (want > nch) want = nch;
    if (want < 1) want = 1;
    seg_chunks = nch > 0 ? (nch + want - 1) / want : 1;
    nseg = nch > 0 ? (nch + seg_chunks - 1) / seg_chunks : 1;
}

// workspace regions start on 256-byte boundaries
static size_t up(size_t x) { return (x + 255) / 256 * 256; }

size_t causal_work_bytes(int B, int H, int N, int du) {
    const size_t nls = (static_cast<size_t>(N) + kLogitSeg - 1) / kLogitSeg;
    const size_t nch = (static_cast<size_t>(N) + kC - 1) / kC;
    const size_t bh = static_cast<size_t>(B) * H;
    int nseg, seg_chunks;
    seg_plan(B, H, N, nseg, seg_chunks);
    return up(bh * N * 4) + up(bh * nls * du * 4) + up(bh * nch * 16) + up(bh * nseg * 16) +
           up(bh * (nseg - 1) * size_t(3) * du * du * 4) + up(size_t(kC) * du * 2) + bh * nch * sizeof(Coef);
}

CausalWork causal_work_carve(void *base, int B, int H, int N, int du) {
    const size_t nls = (static_cast<size_t>(N) + kLogitSeg - 1) / kLogitSeg;
    const size_t nch = (static_cast<size_t>(N) + kC - 1) / kC;
    const size_t bh = static_cast<size_t>(B) * H;
    CausalWork w;
    seg_plan(B, H, N, w.nseg, w.seg_chunks);
    char *b = static_cast<char *>(base);
    w.s = reinterpret_cast<float *>(b);
    b += up(bh * N * 4);
    w.useg = reinterpret_cast<float *>(b);
    b += up(bh * nls * du * 4);
    w.agg = reinterpret_cast<float4 *>(b);
    b += up(bh * nch * 16);
    w.segsc = reinterpret_cast<float4 *>(b);
    b += up(bh * w.nseg * 16);
    w.segst = reinterpret_cast<float *>(b);
    b += up(bh * (w.nseg - 1) * size_t(3) * du * du * 4);
    w.sink = reinterpret_cast<uint16_t *>(b);
    b += up(size_t(kC) * du * 2);
    w.coef = reinterpret_cast<Coef *>(b);
    return w;
}

hipError_t launch_causal_mfma(const Problem &p, const CausalWork &w, hipStream_t stream) {
    hipError_t err = launch_logits(p, w.useg, w.s, w.agg, stream);
    if (err != hipSuccess) return err;
    if (p.d == 128) return p.rope ? launch_one<128, true>(p, w, stream) : launch_one<128, false>(p, w, stream);
    if (p.d == 64) return p.rope ? launch_one<64, true>(p, w, stream) : launch_one<64, false>(p, w, stream);
    return hipErrorInvalidValue;
}

}  // namespace zeros
