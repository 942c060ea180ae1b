// Causal ZeroS forward on the matrix cores: bfloat16 q/k/v with float32 states, d in {64, 128}.
//
// Method: Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计
// (zero-sum weights w_{t,i} = alpha_t e^{s_i} + beta_t s_i + gamma_t after expanding the gated
// first-order and residual terms; angular factor q^_t . k^_i with RoPE as a relative rotation;
// the prefix states of the linear-time scan). The logits s_i and per-chunk logit aggregates come
// from logits.hip. The sequence is cut into chunks of kC = 64 tokens.
//
// causal_prep_kernel, one workgroup per (batch, head, chunk), all chunks in parallel: everything
//   that depends on the tokens of a chunk but not on the value columns, done once per head:
//   the logit carry at the chunk start (combining the aggregates of the earlier chunks), the
//   chunk's scalar scan and coefficients, unit (RoPE-rotated) q^ and k^, A^T = K Q^T on MFMA and
//   the intra-chunk weights W_{t,i} = A (a_t e^{s_i-m_t} + b_t s_i + g_t), i <= t. It writes them
//   to a per-chunk record already laid out as MFMA operands (q^, k^T, W) plus the coefficients.
// causal_main_kernel, one workgroup of 8 waves per (batch, head, 16-column tile of v/o), walks the
//   chunks in order. Waves 0-3 (queries [16w, 16w+16)): o^T = V^T W^T + q^-weighted carried
//   states, on MFMA. Waves 4-7 (state rows [(w-4) d/4, (w-3) d/4)): X, Y, H advanced to the chunk
//   end, K^T V' on MFMA. The W accumulator layout of the prep kernel is the B-operand layout of
//   V^T W^T up to a permutation of the contraction index, which V^T is read with.
// States are kept in a centred basis, X = F/E - H/t0 and Y = G - (P/t0) H. Both have zero-sum
// weights, so they stay of the size of the output, and rounding them (and the update operands)
// to bfloat16 for the MFMA is not amplified by the cancellation between alpha F, beta G and
// gamma H. With RoPE, q^ and k^ are rotated by their absolute position (the angle of the chunk
// start composed with the tabulated angle of the offset inside the chunk), so the carried states
// are in the absolute frame and need no re-basing between chunks.
#include <hip/hip_bf16.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace zeros {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kC = 64;          // tokens per chunk
constexpr int kTile = 16;       // value columns per workgroup
constexpr int kPad = 8;         // bf16 elements of row padding in LDS
constexpr int kRing = 3;        // chunks whose operands are in flight in the scan kernel

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two floats to a packed bfloat16 pair (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    const f32x2v f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    bf16x8 r;
    r[0] = static_cast<short>(a & 0xffff); r[1] = static_cast<short>(a >> 16);
    r[2] = static_cast<short>(b & 0xffff); r[3] = static_cast<short>(b >> 16);
    r[4] = static_cast<short>(c & 0xffff); r[5] = static_cast<short>(c >> 16);
    r[6] = static_cast<short>(d & 0xffff); r[7] = static_cast<short>(d >> 16);
    return r;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, float acc) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v v = *reinterpret_cast<const bf16x2v *>(&a);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

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
// Inputs: the chunk's logits and gate pre-activations in lanes; the carry (m0, E0, P0) at t0,
// updated to the chunk end on return. The sums of e^{s} use the chunk-end maximum M1 as a fixed
// reference (plain prefix sums); when the running maximum rises by more than e^60 inside the
// chunk, an exact (max, sum) scan is used instead so that nothing under- or overflows.
__device__ __forceinline__ void chunk_scan(Coef &cf, int lane, int t0, int nval, float sr_in, float g1v,
                                           float ghv, float &m0, float &E0, float &P0) {
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
        cf.qg[r] = -d1 * (Pt * itt) * itt - sh * itt;
        if (t0 > 0) {
            const float dt = tt - t0f;
            cf.qcx[r] = a * E0p;
            cf.qkap[r] = sh * __fdividef(E0p * dt - t0f * dE, Et * tt * t0f) +
                         d1 * __fdividef(P0 * dt - t0f * pp, tt * tt * t0f);
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
// [ W operands   : 4 query blocks x 2 key-block pairs x 64 lanes x 16 B ]
// [ coefficients : cX, beta, kappa per query; w_X, w_Y per key; rX, cHX, cHY, m1, E1, P1 ]
constexpr int kCoefFloats = 5 * kC + 8;
template <int D> struct Rec {
    static constexpr int KS = D / 32;
    static constexpr size_t q_off = 0;
    static constexpr size_t k_off = q_off + size_t(4) * KS * 1024;
    static constexpr size_t w_off = k_off + size_t(D / 16) * 2 * 1024;
    static constexpr size_t c_off = w_off + size_t(8) * 1024;
    static constexpr size_t bytes = c_off + 1536;
};
enum { kCoCX = 0, kCoBeta = kC, kCoKap = 2 * kC, kCoWX = 3 * kC, kCoWY = 4 * kC, kCoChunk = 5 * kC };

__device__ __forceinline__ void st16(unsigned char *p, const bf16x8 &v) { *reinterpret_cast<bf16x8 *>(p) = v; }
__device__ __forceinline__ bf16x8 ld16(const unsigned char *p) { return *reinterpret_cast<const bf16x8 *>(p); }

constexpr int kPrepThreads = 256;
constexpr int kMainThreads = 512;

template <int D>
struct alignas(16) PSmem {
    alignas(16) uint16_t qh[kC][D + kPad];     // unit (rotated) q rows, bf16
    alignas(16) uint16_t kh[kC][D + kPad];     // unit (rotated) k rows, 16-byte blocks swizzled
    Coef cf;
    float2 rot0[D / 2];                        // cos, sin of t0 * theta_j (chunk start)
};

// cos, sin of r * theta_j for the in-chunk offsets r in [0, kC) and feature pairs j in [0, D/2):
// the rotations the prep kernel applies to q and k (every chunk uses the same table).
template <int D>
__global__ __launch_bounds__(256) void rope_table_kernel(float2 *tab, float base) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= kC * (D / 2)) return;
    const int r = idx / (D / 2), j = idx % (D / 2);
    float c, s;
    rope_cos_sin(rope_rev_per_pos(j, D, base), r, c, s);
    tab[idx] = make_float2(c, s);
}

template <int D, bool ROPE>
__global__ __launch_bounds__(kPrepThreads) void causal_prep_kernel(Problem p, CausalWork work) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PSmem<D> &sm = *reinterpret_cast<PSmem<D> *>(smem_raw);
    using R = Rec<D>;
    constexpr int KS = D / 32;
    constexpr int RT = D / 64;
    constexpr int QW = D / 4;           // features per thread in the load phase
    constexpr int NV = QW / 8;
    constexpr int NP = QW / 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int N = p.N;
    const int nch = (N + kC - 1) / kC;
    const int c = blockIdx.x % nch;
    const int bh = blockIdx.x / nch;
    const int t0 = c * kC, nval = min(kC, N - t0);
    const size_t row0 = static_cast<size_t>(bh) * N;
    unsigned char *rec = work.rec + (static_cast<size_t>(bh) * nch + c) * R::bytes;

    if (ROPE) {
        if (tid < D / 2) {
            float c0, s0;
            rope_cos_sin(rope_rev_per_pos(tid, D, p.rope_base), t0, c0, s0);
            sm.rot0[tid] = make_float2(c0, s0);
        }
        __syncthreads();
    }

    // ---- wave 0: logit carry at t0 from the earlier chunks, then this chunk's scan
    if (wave == 0) {
        float m = kNegInf, e = 0.f, ps = 0.f;
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
        chunk_scan(sm.cf, lane, t0, nval, sv, g1v, ghv, m0, E0, P0);
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
            st16(rec + R::q_off + (size_t(tb * KS + ks) * 64 + lane) * 16, qop[ks]);
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
            st16(rec + R::w_off + (size_t(tb * 2 + pi) * 64 + lane) * 16, as_bf16x8(wv[0], wv[1], wv[2], wv[3]));
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
        co[kCoCX + tid] = sm.cf.qcx[tid];
        co[kCoBeta + tid] = sm.cf.qb[tid];
        co[kCoKap + tid] = sm.cf.qkap[tid];
        co[kCoWX + tid] = sm.cf.wx[tid];
        co[kCoWY + tid] = sm.cf.wy[tid];
        if (tid < 6) {
            const int src[6] = {3, 4, 5, 0, 1, 2};   // rX, cHX, cHY, m1, E1, P1
            co[kCoChunk + tid] = sm.cf.chunk[src[tid]];
        }
    }
}

template <int D>
struct alignas(16) MSmem {
    // v tile, transposed: vt[m][token] (also the H update operand), and the update operands
    // v * w_X, v * w_Y (transposed); double-buffered, the next chunk is staged during this one
    alignas(16) uint16_t vt[2][kTile][kC + kPad];
    alignas(16) uint16_t vx[2][kTile][kC + kPad];
    alignas(16) uint16_t vy[2][kTile][kC + kPad];
    alignas(16) uint16_t st[2][3][kTile][D + kPad];  // X, Y, H transposed, bf16, double-buffered
};

template <int D, bool ROPE>
__global__ __launch_bounds__(kMainThreads) void causal_main_kernel(Problem p, CausalWork work) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    MSmem<D> &sm = *reinterpret_cast<MSmem<D> *>(smem_raw);
    using R = Rec<D>;
    constexpr int NTILE = D / kTile;
    constexpr int KS = D / 32;
    constexpr int RT = D / 64;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int l16 = lane & 15, g4 = lane >> 4;
    const bool qgroup = wave < 4;
    const int wb = wave & 3;

    const int G = gridDim.x;
    int L = blockIdx.x;
    if ((G & 7) == 0) L = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int tile = L % NTILE;
    const int bh = L / NTILE;
    const int N = p.N;
    const int nch = (N + kC - 1) / kC;
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + row0 * D;
    uint16_t *og = static_cast<uint16_t *>(p.o) + row0 * D;
    const unsigned char *rec0 = work.rec + static_cast<size_t>(bh) * nch * R::bytes;

    // staging coordinates: token lr of the chunk, value columns 2*p8 + {0, 1}
    const int lr = tid >> 3, p8 = tid & 7;

    f32x4 X[RT], Y[RT], Hm[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[rt][i] = Y[rt][i] = Hm[rt][i] = 0.f;

    // MFMA operands of a chunk, NOP 16-byte slots per lane. Waves 0-3: slots 0..KS-1 = q^ (query
    // block wb), KS, KS+1 = W (key-block pairs); waves 4-7: slots 0..2RT-1 = k^T (row tiles of
    // wave wb-4, two key steps), the rest repeat slot 0. The loads are the same code in every wave,
    // only the addresses differ.
    constexpr int NOP = KS + 2;
    uint32_t opoff[NOP];
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
        size_t o;
        if (qgroup) o = i < KS ? R::q_off + size_t(wb * KS + i) * 1024 : R::w_off + size_t(wb * 2 + i - KS) * 1024;
        else { const int j = i < 2 * RT ? i : 0; o = R::k_off + size_t((RT * wb + j / 2) * 2 + (j & 1)) * 1024; }
        opoff[i] = static_cast<uint32_t>(o + lane * 16);
    }
    // three scalars per lane: (cX, beta, kappa) of the lane's query in waves 0-3,
    // (rX, cHX, cHY) of the chunk in waves 4-7
    const int tq_lane = 16 * wb + l16;
    const int sc_off0 = qgroup ? kCoCX + tq_lane : kCoChunk + 0;
    const int sc_off1 = qgroup ? kCoBeta + tq_lane : kCoChunk + 1;
    const int sc_off2 = qgroup ? kCoKap + tq_lane : kCoChunk + 2;
    const int tok_lane = lr & ~1;
    const size_t vcol = static_cast<size_t>(tile) * kTile + 2 * p8;

    // Everything one chunk needs from memory, per lane. The record and v of chunk c are read
    // kRing chunks before c is processed (a ring of register slots, the loop unrolled by kRing),
    // so that the latency of the first touch of a record line is covered by the work of the
    // chunks in between.
    struct Slot {
        bf16x8 op[NOP];
        float sc0, sc1, sc2;
        uint32_t pv;           // v of token lr, columns 2*p8 (low) and 2*p8+1
        bool pv_ok;            // token lr exists (else pv is a stand-in row)
        float2 wx2, wy2;       // w_X, w_Y of tokens (lr & ~1), (lr | 1)
    };
    auto load = [&](Slot &sl, const int c) __attribute__((always_inline)) {
        const unsigned char *rec_ = rec0 + static_cast<size_t>(c) * R::bytes;
        const float *co_ = reinterpret_cast<const float *>(rec_ + R::c_off);
#pragma unroll
        for (int i = 0; i < NOP; ++i) sl.op[i] = ld16(rec_ + opoff[i]);
        sl.sc0 = co_[sc_off0];
        sl.sc1 = co_[sc_off1];
        sl.sc2 = co_[sc_off2];
        const int tok_ = c * kC + lr;       // rows past N read row N-1 (in bounds), then zeroed
        sl.pv = *reinterpret_cast<const uint32_t *>(vg + static_cast<size_t>(min(tok_, N - 1)) * D + vcol);
        sl.pv_ok = tok_ < N;                // applied when staging, so the load is not waited for
        sl.wx2 = *reinterpret_cast<const float2 *>(co_ + kCoWX + tok_lane);
        sl.wy2 = *reinterpret_cast<const float2 *>(co_ + kCoWY + tok_lane);
    };

    // stage the v tile of a chunk (transposed token pairs) and its update operands into buffer b
    auto stage = [&](const Slot &sl, const int b) __attribute__((always_inline)) {
        const uint32_t pvv = sl.pv_ok ? sl.pv : 0u;
        const uint32_t other = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(pvv), kRowRor + 8, 0xf, 0xf, false));
        const bool odd = lr & 1;
        const uint32_t pair = odd ? ((other >> 16) | (pvv & 0xffff0000u)) : ((pvv & 0xffffu) | (other << 16));
        const int col = 2 * p8 + (odd ? 1 : 0), tok = lr & ~1;
        const float v0 = lo_f(pair), v1 = hi_f(pair);
        *reinterpret_cast<uint32_t *>(&sm.vt[b][col][tok]) = pair;
        *reinterpret_cast<uint32_t *>(&sm.vx[b][col][tok]) = pack2(v0 * sl.wx2.x, v1 * sl.wx2.y);
        *reinterpret_cast<uint32_t *>(&sm.vy[b][col][tok]) = pack2(v0 * sl.wy2.x, v1 * sl.wy2.y);
    };

    // One chunk: compute with slot sl (chunk ci, staged in buffer ci & 1), stage chunk ci + 1 from
    // slot nx into the other buffer, refill sl, then a single barrier.
    auto body = [&](Slot &sl, const Slot &nx, const int ci) __attribute__((always_inline)) {
        const int t0 = ci * kC;
        const int nval = min(kC, N - t0);
        const int vb = ci & 1;

        const float s0c = sl.sc0, s1c = sl.sc1, s2c = sl.sc2;
        if (qgroup) {
            const int tb = wb;
            const int tq = 16 * tb + l16;
            f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
            // intra-chunk: o^T += V^T W^T over key-block pairs (0,1) and (2,3)
#pragma unroll
            for (int pi = 0; pi < 2; ++pi) {
                if (2 * pi > tb) continue;
                const int kb0 = 2 * pi, kb1 = 2 * pi + 1;
                const uint2 va = *reinterpret_cast<const uint2 *>(&sm.vt[vb][l16][16 * kb0 + 4 * g4]);
                const uint2 vc = (kb1 <= tb) ? *reinterpret_cast<const uint2 *>(&sm.vt[vb][l16][16 * kb1 + 4 * g4])
                                             : make_uint2(0, 0);
                oacc = mfma(as_bf16x8(va.x, va.y, vc.x, vc.y), sl.op[KS + pi], oacc);
            }
            // carried states
            if (t0 > 0) {
                const int sb = ci & 1;
                f32x4 ax = {0.f, 0.f, 0.f, 0.f}, ay = ax, ah = ax;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    ax = mfma(*reinterpret_cast<const bf16x8 *>(&sm.st[sb][0][l16][32 * ks + 8 * g4]), sl.op[ks], ax);
                    ay = mfma(*reinterpret_cast<const bf16x8 *>(&sm.st[sb][1][l16][32 * ks + 8 * g4]), sl.op[ks], ay);
                    ah = mfma(*reinterpret_cast<const bf16x8 *>(&sm.st[sb][2][l16][32 * ks + 8 * g4]), sl.op[ks], ah);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[i] += s0c * ax[i] + s1c * ay[i] + s2c * ah[i];   // cX, beta, kappa
            }
            if (tq < nval) {
                const uint2 ov = make_uint2(pack2(oacc[0], oacc[1]), pack2(oacc[2], oacc[3]));
                *reinterpret_cast<uint2 *>(og + static_cast<size_t>(t0 + tq) * D + tile * kTile + 4 * g4) = ov;
            }
        } else if (ci < nch) {              // padding chunks past the end leave the states alone
            if (t0 > 0) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        X[rt][i] = s0c * X[rt][i] + s1c * Hm[rt][i];   // rX, cHX
                        Y[rt][i] = Y[rt][i] + s2c * Hm[rt][i];           // cHY
                    }
            }
#pragma unroll
            for (int ks2 = 0; ks2 < kC / 32; ++ks2) {
                const int kk0 = 32 * ks2 + 8 * g4;
                const bf16x8 BX = *reinterpret_cast<const bf16x8 *>(&sm.vx[vb][l16][kk0]);
                const bf16x8 BY = *reinterpret_cast<const bf16x8 *>(&sm.vy[vb][l16][kk0]);
                const bf16x8 BH = *reinterpret_cast<const bf16x8 *>(&sm.vt[vb][l16][kk0]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    X[rt] = mfma(sl.op[2 * rt + ks2], BX, X[rt]);
                    Y[rt] = mfma(sl.op[2 * rt + ks2], BY, Y[rt]);
                    Hm[rt] = mfma(sl.op[2 * rt + ks2], BH, Hm[rt]);
                }
            }
            const int nb = (ci + 1) & 1;        // the query waves read st[ci & 1] meanwhile
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int jc = 16 * (RT * wb + rt) + 4 * g4;
                *reinterpret_cast<uint2 *>(&sm.st[nb][0][l16][jc]) = make_uint2(pack2(X[rt][0], X[rt][1]), pack2(X[rt][2], X[rt][3]));
                *reinterpret_cast<uint2 *>(&sm.st[nb][1][l16][jc]) = make_uint2(pack2(Y[rt][0], Y[rt][1]), pack2(Y[rt][2], Y[rt][3]));
                *reinterpret_cast<uint2 *>(&sm.st[nb][2][l16][jc]) = make_uint2(pack2(Hm[rt][0], Hm[rt][1]), pack2(Hm[rt][2], Hm[rt][3]));
            }
        }
        stage(nx, vb ^ 1);
        // this slot is consumed: refill it with the chunk kRing ahead. The load is unconditional
        // (past the end it repeats the last chunk) so that the wait before each use of a slot is
        // a fixed count of younger loads and the other slots stay in flight.
        load(sl, min(ci + kRing, nch - 1));
        lds_barrier();            // chunk done: next staging and states visible, old buffers free
    };

    Slot s0, s1, s2;
    static_assert(kRing == 3, "the loop below is unrolled for a ring of three slots");
    if (nch > 0) {
        // issued in slot order (the empty asm keeps the compiler from reordering them), so that
        // slot 0 is the oldest at the loop entry as it is on every later iteration
        load(s0, 0);
        asm volatile("" ::: "memory");
        load(s1, min(1, nch - 1));
        asm volatile("" ::: "memory");
        load(s2, min(2, nch - 1));
        asm volatile("" ::: "memory");
        stage(s0, 0);
        lds_barrier();
        // whole groups of kRing chunks; a chunk index past the end stores nothing (nval <= 0)
        for (int ci = 0; ci < nch; ci += kRing) {
            body(s0, s1, ci);
            body(s1, s2, ci + 1);
            body(s2, s0, ci + 2);
        }
    }

    // ---- final state (update waves): back to F = E (X + H/t), G = Y + (P/t) H
    if (p.st.F != nullptr) {
        float m0 = kNegInf, E0 = 0.f, P0 = 0.f;
        if (N > 0) {
            const float *co = reinterpret_cast<const float *>(rec0 + static_cast<size_t>(nch - 1) * R::bytes + R::c_off);
            m0 = co[kCoChunk + 3];
            E0 = co[kCoChunk + 4];
            P0 = co[kCoChunk + 5];
        }
        if (!qgroup) {
            const size_t mat0 = static_cast<size_t>(bh) * D * D;
            const float tf = static_cast<float>(N);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float F[4], Gv[4], Hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float hh = Hm[rt][i];
                    F[i] = N > 0 ? E0 * (X[rt][i] + hh / tf) : 0.f;
                    Gv[i] = N > 0 ? Y[rt][i] + (P0 / tf) * hh : 0.f;
                    Hv[i] = hh;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = 16 * (RT * wb + rt) + 4 * g4 + i;
                    const size_t idx = mat0 + static_cast<size_t>(j) * D + tile * kTile + l16;
                    p.st.F[idx] = F[i];
                    p.st.G[idx] = Gv[i];
                    p.st.Hs[idx] = Hv[i];
                }
            }
        }
        if (tile == 0) {
            const int nseg = (N + kLogitSeg - 1) / kLogitSeg;
            if (tid < D) {
                float su = 0.f;
                for (int sg = 0; sg < nseg; ++sg) su += work.useg[(static_cast<size_t>(bh) * nseg + sg) * D + tid];
                p.st.Su[static_cast<size_t>(bh) * D + tid] = su;
            }
            if (tid == 0) {
                p.st.m[bh] = m0;
                p.st.E[bh] = E0;
                p.st.P[bh] = P0;
                p.st.t[bh] = N;
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
    static bool attr_set = false;   // idempotent; a race only repeats the same calls
    if (!attr_set) {
        hipError_t err = set_smem(&causal_prep_kernel<D, ROPE>, sizeof(PSmem<D>));
        if (err == hipSuccess) err = set_smem(&causal_main_kernel<D, ROPE>, sizeof(MSmem<D>));
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    const int nch = (p.N + kC - 1) / kC;
    if (ROPE && nch > 0) {
        hipLaunchKernelGGL((rope_table_kernel<D>), dim3((kC * (D / 2) + 255) / 256), dim3(256), 0, stream,
                           w.rope, p.rope_base);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (nch > 0) {
        hipLaunchKernelGGL((causal_prep_kernel<D, ROPE>), dim3(p.B * p.H * nch), dim3(kPrepThreads),
                           sizeof(PSmem<D>), stream, p, w);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((causal_main_kernel<D, ROPE>), dim3(p.B * p.H * (D / kTile)), dim3(kMainThreads),
                       sizeof(MSmem<D>), stream, p, w);
    return hipGetLastError();
}

}  // namespace

size_t causal_rec_bytes(int d) { return d == 128 ? Rec<128>::bytes : Rec<64>::bytes; }

size_t causal_work_bytes(int B, int H, int N, int du) {
    const size_t a = 256;
    auto up = [a](size_t x) { return (x + a - 1) / a * a; };
    const size_t nseg = (static_cast<size_t>(N) + kLogitSeg - 1) / kLogitSeg;
    const size_t nch = (static_cast<size_t>(N) + kC - 1) / kC;
    const size_t bh = static_cast<size_t>(B) * H;
    return up(bh * N * 4) + up(bh * nseg * du * 4) + up(bh * nch * 16) + up(size_t(kC) * (du / 2) * 8) +
           bh * nch * causal_rec_bytes(du);
}

CausalWork causal_work_carve(void *base, int B, int H, int N, int du) {
    const size_t a = 256;
    auto up = [a](size_t x) { return (x + a - 1) / a * a; };
    const size_t nseg = (static_cast<size_t>(N) + kLogitSeg - 1) / kLogitSeg;
    const size_t nch = (static_cast<size_t>(N) + kC - 1) / kC;
    const size_t bh = static_cast<size_t>(B) * H;
    char *b = static_cast<char *>(base);
    CausalWork w;
    w.s = reinterpret_cast<float *>(b);
    b += up(bh * N * 4);
    w.useg = reinterpret_cast<float *>(b);
    b += up(bh * nseg * du * 4);
    w.agg = reinterpret_cast<float4 *>(b);
    b += up(bh * nch * 16);
    w.rope = reinterpret_cast<float2 *>(b);
    b += up(size_t(kC) * (du / 2) * 8);
    w.rec = reinterpret_cast<unsigned char *>(b);
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
