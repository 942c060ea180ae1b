// Causal ZeroS forward on the matrix cores: bfloat16 q/k/v with float32 states, d in {64, 128}.
//
// Method: Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计
// (zero-sum weights w_{t,i} = alpha_t e^{s_i} + beta_t s_i + gamma_t after expanding the gated
// first-order and residual terms; angular factor q^_t . k^_i with RoPE as a relative rotation;
// the prefix states of the linear-time scan). The optional zero-order gate of the same section
// (a first layer may keep the uniform term) adds sigma0_t/t to gamma_t. The logits s_i and per-chunk logit aggregates come
// from logits.hip. The sequence is cut into chunks of kC = 64 tokens.
//
// causal_prep_kernel, one workgroup per (batch, head, chunk), all chunks in parallel: everything
//   that depends on the tokens of a chunk but not on the value columns, done once per head:
//   the logit carry at the chunk start (combining the aggregates of the earlier chunks), the
//   chunk's scalar scan and coefficients, unit (RoPE-rotated) q^ and k^, A^T = K Q^T on MFMA and
//   the intra-chunk weights W_{t,i} = A (a_t e^{s_i-m_t} + b_t s_i + g_t), i <= t. It writes them
//   to a per-chunk record already laid out as MFMA operands (q^, k^T, W) plus the coefficients.
// causal_seg_kernel, one workgroup of d/16 waves per (batch, head, segment of the chunks), walks
//   its chunks in order; wave w owns value columns [16w, 16w+16) and all d rows of X, Y, H in
//   float32 registers. Per chunk: o^T = S^T Q^T (carried states, S^T straight from the registers)
//   + V^T W^T (intra-chunk), then the states advance to the chunk end with K^T V' on MFMA. The W
//   accumulator layout of the prep kernel is the B-operand layout of V^T W^T up to a permutation
//   of the contraction index, which V^T is read with. Segments are chained exactly by a pass over
//   each segment from a zero state and a combine step (see the segment-parallel scan below).
// States are kept in a centred basis, X = F/E - H/t0 and Y = G - (P/t0) H. Both have zero-sum
// weights, so they stay of the size of the output, and rounding them (and the update operands)
// to bfloat16 for the MFMA is not amplified by the cancellation between alpha F, beta G and
// gamma H. With RoPE, q^ and k^ are rotated by their absolute position (the angle of the chunk
// start composed with the tabulated angle of the offset inside the chunk), so the carried states
// are in the absolute frame and need no re-basing between chunks.
#include <hip/hip_bf16.h>

#include <atomic>

#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace zeros {
namespace {

constexpr int kC = 64;          // tokens per chunk
constexpr int kTile = 16;       // value columns per workgroup
constexpr int kPad = 8;         // bf16 elements of row padding in LDS

// Per-chunk coefficients, produced one chunk ahead by wave 0 (double-buffered).
struct Coef {
    float qa[kC], qm[kC], qb[kC], qg[kC], qcx[kC], qkap[kC];   // per query t
    float wx[kC], wy[kC], s[kC], ek[kC];                        // per key i; ek = e^{s_i - m1}
    float chunk[8];                      // m1, E1, P1, rX, cHX, cHY, exact-exp flag
};

// Column-block swizzle of the k rows in LDS: 16-byte block b of row `key` is stored at
// b ^ kswz(key), so the 8-key column gathers hit distinct LDS banks.
__device__ __forceinline__ int kswz(int key) { return ((key >> 3) & 3) << 1; }

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


// ---- per-chunk record written by the prep kernel and read by the main kernel ------------------
// [ Q^ operands  : 4 query blocks x KS k-steps x 64 lanes x 16 B ]
// [ K^T operands : d/16 row tiles x 2 key steps x 64 lanes x 16 B ]
// [ W operands   : (query block tb, key-block pair pi) with 2 pi <= tb, the six that the causal mask
//                  leaves non-zero, x 64 lanes x 16 B; piece index w_piece(tb, pi) ]
// [ coefficients : (cX, beta, kappa, 0) per query; (w_X, w_Y) per key; rX, cHX, cHY, m1, E1, P1 ]
template <int D> struct Rec {
    static constexpr int KS = D / 32;
    static constexpr size_t q_off = 0;
    static constexpr size_t k_off = q_off + size_t(4) * KS * 1024;
    static constexpr size_t w_off = k_off + size_t(D / 16) * 2 * 1024;
    static constexpr size_t c_off = w_off + size_t(6) * 1024;
    static constexpr size_t bytes = c_off + (6 * kC + 8) * 4;
};
enum { kCoQ = 0, kCoW = 4 * kC, kCoChunk = 6 * kC };   // float offsets in the coefficient block
// W piece of query block tb (0..3) and key-block pair pi (keys 32 pi .. 32 pi + 31), 2 pi <= tb
__device__ __forceinline__ int w_piece(int tb, int pi) { return tb < 2 ? tb : 2 * tb - 2 + pi; }

__device__ __forceinline__ void st16(unsigned char *p, const bf16x8 &v) { *reinterpret_cast<bf16x8 *>(p) = v; }
__device__ __forceinline__ bf16x8 ld16(const unsigned char *p) { return *reinterpret_cast<const bf16x8 *>(p); }

constexpr int kPrepThreads = 256;

template <int D>
struct alignas(16) PSmem {
    alignas(16) uint16_t qh[kC][D + kPad];     // unit (rotated) q rows, bf16
    alignas(16) uint16_t kh[kC][D + kPad];     // unit (rotated) k rows, 16-byte blocks swizzled
    Coef cf;
    float2 rot0[D / 2];                        // cos, sin of t0 * theta_j (chunk start)
};

template <int D, bool ROPE>
__global__ __launch_bounds__(kPrepThreads) void causal_prep_kernel(Problem p, CausalWork work) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PSmem<D> &sm = *reinterpret_cast<PSmem<D> *>(smem_raw);
    using R = Rec<D>;
    constexpr int KS = D / 32;
    constexpr int RT = D / 64;
    constexpr int QW = D / 4;           // features per thread in the load phase
    constexpr int NV = QW / 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int N = p.N;
    const int nch = (N + kC - 1) / kC;
    const int c = blockIdx.x % nch;
    const int bh = blockIdx.x / nch;
    const int t0 = c * kC, nval = min(kC, N - t0);
    const size_t row0 = static_cast<size_t>(bh) * N;
    unsigned char *rec = work.rec + (static_cast<size_t>(bh) * nch + c) * R::bytes;
    // a sequence continued from a state: its tokens are positions tin + 1 ...
    const bool cont = p.sin.F != nullptr;
    const int tin = cont ? p.sin.t[bh] : 0;

    if (ROPE) {
        if (tid < D / 2) {
            float c0, s0;
            rope_cos_sin(rope_rev_per_pos(tid, D, p.rope_base), tin + t0, c0, s0);
            sm.rot0[tid] = make_float2(c0, s0);
        }
        __syncthreads();
    }

    // ---- wave 0: logit carry at t0 from the state (if any) and the earlier chunks, then this
    // chunk's scan
    if (wave == 0) {
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
        chunk_scan(sm.cf, lane, tin + t0, nval, sv, g1v, ghv, s0, m0, E0, P0);
    }

    // ---- unit q^, k^ rows, rotated by their offset inside the chunk
    {
        const int lr = tid >> 2, f0 = (tid & 3) * QW;
        const bool valid = lr < nval;
        const size_t base = (row0 + t0 + lr) * D + f0;
        const uint16_t *qg = static_cast<const uint16_t *>(p.q), *kg = static_cast<const uint16_t *>(p.k);
        uint4 pq[NV], pk[NV];
#pragma unroll
        for (int a = 0; a < NV; ++a) {
            pq[a] = valid ? *reinterpret_cast<const uint4 *>(qg + base + 8 * a) : make_uint4(0, 0, 0, 0);
            pk[a] = valid ? *reinterpret_cast<const uint4 *>(kg + base + 8 * a) : make_uint4(0, 0, 0, 0);
        }
        float ssq = 0.f, ssk = 0.f;
#pragma unroll
        for (int a = 0; a < NV; ++a) {
            ssq = dot2_bf16(pq[a].x, ssq); ssq = dot2_bf16(pq[a].y, ssq);
            ssq = dot2_bf16(pq[a].z, ssq); ssq = dot2_bf16(pq[a].w, ssq);
            ssk = dot2_bf16(pk[a].x, ssk); ssk = dot2_bf16(pk[a].y, ssk);
            ssk = dot2_bf16(pk[a].z, ssk); ssk = dot2_bf16(pk[a].w, ssk);
        }
        ssq = group_sum<4>(ssq);
        ssk = group_sum<4>(ssk);
        const float iq = valid ? __frsqrt_rn(fmaxf(ssq, 1e-24f)) : 0.f;
        const float ik = valid ? __frsqrt_rn(fmaxf(ssk, 1e-24f)) : 0.f;
#pragma unroll
        for (int a = 0; a < NV; ++a) {
            uint32_t wq[4] = {pq[a].x, pq[a].y, pq[a].z, pq[a].w};
            uint32_t wk[4] = {pk[a].x, pk[a].y, pk[a].z, pk[a].w};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float q0 = lo_f(wq[b]), q1 = hi_f(wq[b]);
                const float k0 = lo_f(wk[b]), k1 = hi_f(wk[b]);
                if (ROPE) {
                    // angle of position t0 + lr = angle of t0 + angle of lr
                    const int jp = f0 / 2 + 4 * a + b;
                    const float2 tr = work.rope[lr * (D / 2) + jp], t0r = sm.rot0[jp];
                    const float cs = t0r.x * tr.x - t0r.y * tr.y, sn = t0r.y * tr.x + t0r.x * tr.y;
                    const float cq = cs * iq, sq = sn * iq, ck = cs * ik, sk = sn * ik;
                    wq[b] = pack2(q0 * cq - q1 * sq, q0 * sq + q1 * cq);
                    wk[b] = pack2(k0 * ck - k1 * sk, k0 * sk + k1 * ck);
                } else {
                    wq[b] = pack2(q0 * iq, q1 * iq);
                    wk[b] = pack2(k0 * ik, k1 * ik);
                }
            }
            const int blk = f0 / 8 + a;
            *reinterpret_cast<uint4 *>(&sm.qh[lr][8 * blk]) = make_uint4(wq[0], wq[1], wq[2], wq[3]);
            *reinterpret_cast<uint4 *>(&sm.kh[lr][8 * (blk ^ kswz(lr))]) = make_uint4(wk[0], wk[1], wk[2], wk[3]);
        }
    }
    __syncthreads();

    // ---- query block tb = wave: q^ operands, A^T tiles, intra-chunk weights
    {
        const int tb = wave;
        const Coef &cf = sm.cf;
        bf16x8 qop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qop[ks] = *reinterpret_cast<const bf16x8 *>(&sm.qh[16 * tb + l16][32 * ks + 8 * g4]);
            // the record holds features {32ks + 4g4 + i, 32ks + 16 + 4g4 + i}, i < 4: the order in
            // which a lane of the scan kernel holds the rows of two 16-row state accumulator tiles
            const uint2 qa = *reinterpret_cast<const uint2 *>(&sm.qh[16 * tb + l16][32 * ks + 4 * g4]);
            const uint2 qc = *reinterpret_cast<const uint2 *>(&sm.qh[16 * tb + l16][32 * ks + 16 + 4 * g4]);
            st16(rec + R::q_off + (size_t(tb * KS + ks) * 64 + lane) * 16, as_bf16x8(qa.x, qa.y, qc.x, qc.y));
        }
        f32x4 at[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) at[kb][i] = 0.f;
            if (kb <= tb) {
                const int key = 16 * kb + l16;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sm.kh[key][8 * ((4 * ks + g4) ^ kswz(key))]);
                    at[kb] = mfma(a, qop[ks], at[kb]);
                }
            }
        }
        const int tq = 16 * tb + l16;
        const float qa = cf.qa[tq], qm = cf.qm[tq], qb = cf.qb[tq], qgm = cf.qg[tq];
        const bool exact_exp = cf.chunk[6] != 0.f;
#pragma unroll
        for (int pi = 0; pi < 2; ++pi) {
            uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int kb = 2 * pi + h2;
                if (kb > tb) continue;
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
                float w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * kb + 4 * g4 + i;
                    const float x = at[kb][i] * (qa * ke_[i] + qb * ks_[i] + qgm);
                    w[i] = (key <= tq && tq < nval) ? x : 0.f;
                }
                wv[2 * h2] = pack2(w[0], w[1]);
                wv[2 * h2 + 1] = pack2(w[2], w[3]);
            }
            if (2 * pi <= tb)
                st16(rec + R::w_off + (size_t(w_piece(tb, pi)) * 64 + lane) * 16, as_bf16x8(wv[0], wv[1], wv[2], wv[3]));
        }
    }

    // ---- k^T operands of the state update: row tiles [RT*wave, RT*wave+RT), 2 key steps
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int jb = RT * wave + rt;
        const int j = 16 * jb + l16;
#pragma unroll
        for (int ks2 = 0; ks2 < kC / 32; ++ks2) {
            const int kk0 = 32 * ks2 + 8 * g4;
            const int jc = (((j >> 3) ^ (2 * g4)) << 3) | (j & 7);   // kswz(kk0 + c) == 2 * g4
            bf16x8 a;
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) a[cc] = static_cast<short>(sm.kh[kk0 + cc][jc]);
            st16(rec + R::k_off + (size_t(jb * 2 + ks2) * 64 + lane) * 16, a);
        }
    }

    // ---- coefficients used by the main kernel
    if (tid < kC) {
        float *co = reinterpret_cast<float *>(rec + R::c_off);
        *reinterpret_cast<float4 *>(co + kCoQ + 4 * tid) = make_float4(sm.cf.qcx[tid], sm.cf.qb[tid], sm.cf.qkap[tid], 0.f);
        *reinterpret_cast<float2 *>(co + kCoW + 2 * tid) = make_float2(sm.cf.wx[tid], sm.cf.wy[tid]);
        if (tid < 8) {
            const int src[8] = {3, 4, 5, 0, 1, 2, 7, 7};   // rX, cHX, cHY, m1, E1, P1, 0, 0
            co[kCoChunk + tid] = tid < 6 ? sm.cf.chunk[src[tid]] : 0.f;
        }
    }
}

// ---- segment-parallel scan ----------------------------------------------------------------
//
// The chunks of a head are cut into nseg segments of seg_chunks chunks. One workgroup of D/16 waves
// owns a whole head (wave w: value columns [16w, 16w+16), all D state rows of X, Y, H in float32
// registers) for one segment, so every record chunk is read once per head.
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

// LDS bytes of one staged record: whole 64-piece (1 KiB) wave copies
template <int D> constexpr int kRecLds = int((Rec<D>::bytes / 16 + 63) / 64 * 64 * 16);

template <int D, bool ROPE, bool PASS1>
__global__ __launch_bounds__(D * 4) void causal_seg_kernel(Problem p, CausalWork work) {
    // Two record buffers as separate objects: the next chunk is copied into one by direct
    // global-to-LDS loads while the other is read, and the compiler can tell the two apart (so
    // it does not wait for the copy before reading the current one).
    __shared__ __align__(16) unsigned char recA[kRecLds<D>];
    __shared__ __align__(16) unsigned char recB[kRecLds<D>];
    // per wave: its v tile transposed, vt[m][token] (also the H update operand), and the update
    // operands v * w_X, v * w_Y, transposed
    __shared__ __align__(16) uint16_t svt[D / 16][kTile][kC + kPad];
    __shared__ __align__(16) uint16_t svx[D / 16][kTile][kC + kPad];
    __shared__ __align__(16) uint16_t svy[D / 16][kTile][kC + kPad];
    using R = Rec<D>;
    constexpr int NW = D / 16;          // waves
    constexpr int NT = NW * 64;
    constexpr int KS = D / 32;          // 32-feature steps of the carried-state products
    constexpr int JB = D / 16;          // 16-row state tiles
    constexpr int kPieces = int(R::bytes / 16);                 // 16-byte pieces of a record

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
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + row0 * D;
    uint16_t *og = static_cast<uint16_t *>(p.o) + row0 * D;
    const unsigned char *rec0 = work.rec + static_cast<size_t>(bh) * nch * R::bytes;
    // a sequence continued from a state: tokens are positions tin + 1 ..., and the first segment
    // of the main pass starts from that state
    const bool cont = p.sin.F != nullptr;
    const int tin = cont ? p.sin.t[bh] : 0;

    // state of this wave's columns: X, Y, H rows 16 jb + 4 g4 + i, column 16 w + l16
    f32x4 X[JB], Y[JB], Hm[JB];
    const size_t sidx = static_cast<size_t>(w) * 64 + lane;       // float4 index inside a (s, jb) block
    if (!PASS1 && seg == 0 && tin > 0) {
        // the given state in the centred basis: X = F/E - H/t, Y = G - (P/t) H
        const size_t mat0 = static_cast<size_t>(bh) * D * D;
        const float iE = 1.f / p.sin.E[bh], it = 1.f / static_cast<float>(tin);
        const float pt = p.sin.P[bh] * it;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t idx = mat0 + static_cast<size_t>(16 * jb + 4 * g4 + i) * D + w * kTile + l16;
                const float hh = p.sin.Hs[idx];
                X[jb][i] = p.sin.F[idx] * iE - hh * it;
                Y[jb][i] = p.sin.G[idx] - pt * hh;
                Hm[jb][i] = hh;
            }
    } else if (!PASS1 && seg > 0) {
        const float4 *st0 = reinterpret_cast<const float4 *>(work.segst + (static_cast<size_t>(bh) * (nseg - 1) + seg - 1) * kSegFloats<D>);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            const float4 a = st0[(size_t(0 * JB + jb) * NW) * 64 + sidx];
            const float4 b = st0[(size_t(1 * JB + jb) * NW) * 64 + sidx];
            const float4 c = st0[(size_t(2 * JB + jb) * NW) * 64 + sidx];
            X[jb] = f32x4{a.x, a.y, a.z, a.w};
            Y[jb] = f32x4{b.x, b.y, b.z, b.w};
            Hm[jb] = f32x4{c.x, c.y, c.z, c.w};
        }
    } else {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int i = 0; i < 4; ++i) X[jb][i] = Y[jb][i] = Hm[jb][i] = 0.f;
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

    // v of this wave's columns: lane holds tokens 2 (lane & 31), +1 and columns 8 (lane >> 5) + [0, 8)
    const int vtok = 2 * (lane & 31), vh = lane >> 5;
    const size_t vcol = static_cast<size_t>(w) * kTile + 8 * vh;
    uint4 va, vb;
    // record pieces [p0, p1) of chunk c into LDS buffer dst at their record offsets (direct copies:
    // wave w moves pieces p0 + 64 w + NT i + lane; lanes past p1 repeat the last piece into the
    // padding of the buffer, which ends on a whole 64-piece copy)
    auto copy_range = [&](const uint4 *src, unsigned char *dst, const int p0, const int p1) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < (p1 - p0 + NT - 1) / NT; ++i) {
            const int base = p0 + w * 64 + i * NT;               // wave-uniform
            if (base < p1)
                __builtin_amdgcn_global_load_lds(src + min(base + lane, p1 - 1), dst + base * 16, 16, 0, 0);
        }
    };
    // v rows of chunk c into registers, and the record parts this pass reads into LDS buffer dst:
    // the whole record for the main pass, the k^T operands and the coefficients for pass 1
    auto fetch = [&](const int c, unsigned char *dst) __attribute__((always_inline)) {
        const int t_ = c * kC + vtok;      // rows past N read row N-1 (in bounds)
        va = *reinterpret_cast<const uint4 *>(vg + static_cast<size_t>(min(t_, N - 1)) * D + vcol);
        vb = *reinterpret_cast<const uint4 *>(vg + static_cast<size_t>(min(t_ + 1, N - 1)) * D + vcol);
        const uint4 *src = reinterpret_cast<const uint4 *>(rec0 + static_cast<size_t>(c) * R::bytes);
        if (PASS1) {
            copy_range(src, dst, int(R::k_off / 16), int(R::w_off / 16));
            copy_range(src, dst, int(R::c_off / 16), kPieces);
        } else {
            copy_range(src, dst, 0, kPieces);
        }
    };

    if (c_begin < c_end) fetch(c_begin, recA);
    // unconditional: the start-state loads and the first copies are complete on every path into
    // the loop, so no wait inside it has to cover them
    __syncthreads();
    auto chunk = [&](const int c, const unsigned char *rb, unsigned char *rn) __attribute__((always_inline)) {
        const int t0 = c * kC;
        const int nval = min(kC, N - t0);
        const bool has_prev = tin + t0 > 0;      // tokens before this chunk (a carried state)
        const float *co = reinterpret_cast<const float *>(rb + R::c_off);
        const float4 ch = *reinterpret_cast<const float4 *>(co + kCoChunk);   // rX, cHX, cHY, m1
        if (has_prev && rho < 0x1p-40f) {        // fold rho into Z (rare; the same on every lane)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                for (int i = 0; i < 4; ++i) X[jb][i] *= rho;
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

        // ---- stage this wave's v tile (token pairs per column) and the update operands
        // v w_X / rho1 and v w_Y
        {
            // rows past N hold copies of row N - 1 (finite); every product they enter is zero: the
            // record's k^ rows and W columns of absent tokens are zero
            const uint32_t a4[4] = {va.x, va.y, va.z, va.w};
            const uint32_t b4[4] = {vb.x, vb.y, vb.z, vb.w};
            const float4 w4 = *reinterpret_cast<const float4 *>(co + kCoW + 2 * vtok);   // wX, wY of both tokens
            const float4 wv = make_float4(w4.x * irho1, w4.y, w4.z * irho1, w4.w);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // columns 8 vh + 2i (low halves) and 8 vh + 2i + 1 (high halves)
                const uint32_t plo = (a4[i] & 0xffffu) | (b4[i] << 16);           // (a.lo, b.lo)
                const uint32_t phi = (a4[i] >> 16) | (b4[i] & 0xffff0000u);       // (a.hi, b.hi)
                const int m0 = 8 * vh + 2 * i;
                *reinterpret_cast<uint32_t *>(&svt[w][m0][vtok]) = plo;
                *reinterpret_cast<uint32_t *>(&svt[w][m0 + 1][vtok]) = phi;
                const float x0 = lo_f(a4[i]), y0 = lo_f(b4[i]), x1 = hi_f(a4[i]), y1 = hi_f(b4[i]);
                *reinterpret_cast<uint32_t *>(&svx[w][m0][vtok]) = pack2(x0 * wv.x, y0 * wv.z);
                *reinterpret_cast<uint32_t *>(&svx[w][m0 + 1][vtok]) = pack2(x1 * wv.x, y1 * wv.z);
                *reinterpret_cast<uint32_t *>(&svy[w][m0][vtok]) = pack2(x0 * wv.y, y0 * wv.w);
                *reinterpret_cast<uint32_t *>(&svy[w][m0 + 1][vtok]) = pack2(x1 * wv.y, y1 * wv.w);
            }
        }

        // ---- carried-state products and the state update, interleaved by pairs of row tiles:
        // step ks reads rows 2ks, 2ks+1 of Z, Y', H (as bf16 MFMA operands, the state at t0), after
        // which those rows are advanced by K^T V' on MFMA.
        // every operand from this wave's staging area is read here, before the next record's
        // copies are issued: afterwards the wave reads only the current record buffer, which the
        // compiler can tell apart from the copy target (no wait for the copies inside the chunk)
        bf16x8 BX[kC / 32], BY[kC / 32], BH[kC / 32];
#pragma unroll
        for (int ks2 = 0; ks2 < kC / 32; ++ks2) {
            const int kk0 = 32 * ks2 + 8 * g4;
            BX[ks2] = *reinterpret_cast<const bf16x8 *>(&svx[w][l16][kk0]);
            BY[ks2] = *reinterpret_cast<const bf16x8 *>(&svy[w][l16][kk0]);
            BH[ks2] = *reinterpret_cast<const bf16x8 *>(&svt[w][l16][kk0]);
        }
        uint2 VA[2], VC[2];                  // V^T operand halves of the intra-chunk product
        if (!PASS1) {
#pragma unroll
            for (int pi = 0; pi < 2; ++pi) {
                VA[pi] = *reinterpret_cast<const uint2 *>(&svt[w][l16][32 * pi + 4 * g4]);
                VC[pi] = *reinterpret_cast<const uint2 *>(&svt[w][l16][32 * pi + 16 + 4 * g4]);
            }
        }
        // next chunk's record and v, in flight during this chunk
        fetch(min(c + 1, c_end - 1), rn);
        f32x4 ax[4], ay[4], ah[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) ax[tb][i] = ay[tb][i] = ah[tb][i] = 0.f;
        const bool carried = !PASS1 && has_prev;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (carried) {
                const f32x4 &x0 = X[2 * ks], &x1 = X[2 * ks + 1];
                const f32x4 &y0 = Y[2 * ks], &y1 = Y[2 * ks + 1];
                const f32x4 &h0 = Hm[2 * ks], &h1 = Hm[2 * ks + 1];
                const bf16x8 AX = as_bf16x8(pack2(x0[0], x0[1]), pack2(x0[2], x0[3]), pack2(x1[0], x1[1]), pack2(x1[2], x1[3]));
                const bf16x8 AY = as_bf16x8(pack2(y0[0], y0[1]), pack2(y0[2], y0[3]), pack2(y1[0], y1[1]), pack2(y1[2], y1[3]));
                const bf16x8 AH = as_bf16x8(pack2(h0[0], h0[1]), pack2(h0[2], h0[3]), pack2(h1[0], h1[1]), pack2(h1[2], h1[3]));
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const bf16x8 Bq = ld16(rb + R::q_off + (size_t(tb * KS + ks) * 64 + lane) * 16);
                    ax[tb] = mfma(AX, Bq, ax[tb]);
                    ay[tb] = mfma(AY, Bq, ay[tb]);
                    ah[tb] = mfma(AH, Bq, ah[tb]);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int jb = 2 * ks + jj;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    X[jb][i] += hz * Hm[jb][i];
                    Y[jb][i] += hy * Hm[jb][i];
                }
#pragma unroll
                for (int ks2 = 0; ks2 < kC / 32; ++ks2) {
                    const bf16x8 Ak = ld16(rb + R::k_off + (size_t(jb * 2 + ks2) * 64 + lane) * 16);
                    X[jb] = mfma(Ak, BX[ks2], X[jb]);
                    Y[jb] = mfma(Ak, BY[ks2], Y[jb]);
                    Hm[jb] = mfma(Ak, BH[ks2], Hm[jb]);
                }
            }
        }
        if (PASS1) {
            // the first chunk of the sequence starts from nothing
            Rs = has_prev ? ch.x * Rs : 0.f;
        } else {
            // ---- outputs: coefficients on the carried-state products, plus V^T W^T (intra-chunk)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f32x4 oacc;
                const float4 cq = *reinterpret_cast<const float4 *>(co + kCoQ + 4 * (16 * tb + l16));  // cX, beta, kappa
                // X = rho Z at t0
                const float cz = cq.x * rho, chh = cq.z;
#pragma unroll
                // (without a carried state the products are zero and the coefficients finite)
                for (int i = 0; i < 4; ++i) oacc[i] = cz * ax[tb][i] + cq.y * ay[tb][i] + chh * ah[tb][i];
#pragma unroll
                for (int pi = 0; pi < 2; ++pi) {
                    if (2 * pi > tb) continue;
                    const uint2 a = VA[pi];
                    const uint2 e = (2 * pi + 1 <= tb) ? VC[pi] : make_uint2(0, 0);
                    const bf16x8 Bw = ld16(rb + R::w_off + (size_t(w_piece(tb, pi)) * 64 + lane) * 16);
                    oacc = mfma(as_bf16x8(a.x, a.y, e.x, e.y), Bw, oacc);
                }
                // rows past the end go to a sink in the workspace: the store is unconditional, so the
                // waits for the next chunk's loads never have to cover an optional store
                const int tq = 16 * tb + l16;
                uint16_t *dst = tq < nval ? og + static_cast<size_t>(t0 + tq) * D : work.sink + static_cast<size_t>(tq) * D;
                const uint2 ov = make_uint2(pack2(oacc[0], oacc[1]), pack2(oacc[2], oacc[3]));
                *reinterpret_cast<uint2 *>(dst + w * kTile + 4 * g4) = ov;
            }
        }
        rho = rho1;
        alp = alp1;
        bet = bet1;
        __syncthreads();          // copies of chunk c + 1 landed (vmcnt) and visible; this buffer free
    };
    for (int c = c_begin; c < c_end; c += 2) {
        chunk(c, recA, recB);
        if (c + 1 < c_end) chunk(c + 1, recB, recA);
    }

    // back to the plain basis: X = rho Z
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[jb][i] *= rho;
    if (PASS1) {
        // segment-local sums and the composed scalar map, for the combine step
        float4 *dst = reinterpret_cast<float4 *>(work.segst + (static_cast<size_t>(bh) * (nseg - 1) + seg) * kSegFloats<D>);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            dst[(size_t(0 * JB + jb) * NW) * 64 + sidx] = make_float4(X[jb][0], X[jb][1], X[jb][2], X[jb][3]);
            dst[(size_t(1 * JB + jb) * NW) * 64 + sidx] = make_float4(Y[jb][0], Y[jb][1], Y[jb][2], Y[jb][3]);
            dst[(size_t(2 * JB + jb) * NW) * 64 + sidx] = make_float4(Hm[jb][0], Hm[jb][1], Hm[jb][2], Hm[jb][3]);
        }
        if (tid == 0) work.segsc[static_cast<size_t>(bh) * nseg + seg] = make_float4(Rs, alp, bet, 0.f);
        return;
    }

    // ---- final recurrent state (last segment): back to F = E (X + H/t), G = Y + (P/t) H
    if (p.st.F != nullptr && seg == nseg - 1) {
        float m0 = kNegInf, E0 = 0.f, P0 = 0.f;
        if (N > 0) {
            const float *co = reinterpret_cast<const float *>(rec0 + static_cast<size_t>(nch - 1) * R::bytes + R::c_off);
            m0 = co[kCoChunk + 3];
            E0 = co[kCoChunk + 4];
            P0 = co[kCoChunk + 5];
        }
        const size_t mat0 = static_cast<size_t>(bh) * D * D;
        const float tf = static_cast<float>(tin + N);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float hh = Hm[jb][i];
                const int j = 16 * jb + 4 * g4 + i;
                const size_t idx = mat0 + static_cast<size_t>(j) * D + w * kTile + l16;
                p.st.F[idx] = N > 0 ? E0 * (X[jb][i] + hh / tf) : 0.f;
                p.st.G[idx] = N > 0 ? Y[jb][i] + (P0 / tf) * hh : 0.f;
                p.st.Hs[idx] = hh;
            }
        const int nls = (N + kLogitSeg - 1) / kLogitSeg;
        if (tid < D) {
            float su = cont ? p.sin.Su[static_cast<size_t>(bh) * D + tid] : 0.f;
            for (int sg = 0; sg < nls; ++sg) su += work.useg[(static_cast<size_t>(bh) * nls + sg) * D + tid];
            p.st.Su[static_cast<size_t>(bh) * D + tid] = su;
        }
        if (tid == 0) {
            p.st.m[bh] = m0;
            p.st.E[bh] = E0;
            p.st.P[bh] = P0;
            p.st.t[bh] = tin + N;
        }
    }
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

template <typename K>
hipError_t set_smem(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(bytes));
}

template <int D, bool ROPE>
hipError_t launch_one(const Problem &p, const CausalWork &w, hipStream_t stream) {
    // the LDS size attribute is per device: set once on each device the library launches on.
    // The flags are atomics, so concurrent first calls from several threads are well defined (both
    // may set the attribute; the call is idempotent).
    constexpr int kMaxDev = 64;
    static std::atomic<bool> attr_set[kMaxDev];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const bool known = dev >= 0 && dev < kMaxDev;
    if (!known || !attr_set[dev].load(std::memory_order_acquire)) {
        err = set_smem(&causal_prep_kernel<D, ROPE>, sizeof(PSmem<D>));
        if (err != hipSuccess) return err;
        if (known) attr_set[dev].store(true, std::memory_order_release);
    }
    const int nch = (p.N + kC - 1) / kC;
    const int bh = p.B * p.H;
    if (nch > 0) {
        hipLaunchKernelGGL((causal_prep_kernel<D, ROPE>), dim3(bh * nch), dim3(kPrepThreads),
                           sizeof(PSmem<D>), stream, p, w);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (w.nseg > 1) {
        hipLaunchKernelGGL((causal_seg_kernel<D, ROPE, true>), dim3(bh * (w.nseg - 1)), dim3(D * 4), 0,
                           stream, p, w);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL((causal_seg_combine_kernel<D>), dim3(bh, (D * D / 4 + 255) / 256), dim3(256), 0,
                           stream, p, w);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    hipLaunchKernelGGL((causal_seg_kernel<D, ROPE, false>), dim3(bh * w.nseg), dim3(D * 4), 0, stream, p, w);
    return hipGetLastError();
}

}  // namespace

size_t causal_rec_bytes(int d) { return d == 128 ? Rec<128>::bytes : Rec<64>::bytes; }

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
    return up(bh * N * 4) + up(bh * nls * du * 4) + up(bh * nch * 16) + up(size_t(kC) * (du / 2) * 8) +
           up(bh * nseg * 16) + up(bh * (nseg - 1) * size_t(3) * du * du * 4) + up(size_t(kC) * du * 2) +
           bh * nch * causal_rec_bytes(du);
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
    w.rope = reinterpret_cast<float2 *>(b);
    b += up(size_t(kC) * (du / 2) * 8);
    w.segsc = reinterpret_cast<float4 *>(b);
    b += up(bh * w.nseg * 16);
    w.segst = reinterpret_cast<float *>(b);
    b += up(bh * (w.nseg - 1) * size_t(3) * du * du * 4);
    w.sink = reinterpret_cast<uint16_t *>(b);
    b += up(size_t(kC) * du * 2);
    w.rec = reinterpret_cast<unsigned char *>(b);
    return w;
}

hipError_t launch_causal_mfma(const Problem &p, const CausalWork &w, hipStream_t stream) {
    hipError_t err = launch_logits(p, w.useg, w.s, w.agg, p.rope ? w.rope : nullptr, stream);
    if (err != hipSuccess) return err;
    if (p.d == 128) return p.rope ? launch_one<128, true>(p, w, stream) : launch_one<128, false>(p, w, stream);
    if (p.d == 64) return p.rope ? launch_one<64, true>(p, w, stream) : launch_one<64, false>(p, w, stream);
    return hipErrorInvalidValue;
}

}  // namespace zeros
