// Causal ZeroS forward on the matrix cores: bfloat16 q/k/v with float32 states, d in {64, 128}.
//
// Method: Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计
// (zero-sum weights w_{t,i} = alpha_t e^{s_i} + beta_t s_i + gamma_t after expanding the gated
// first-order and residual terms; angular factor q^_t . k^_i with RoPE as a relative rotation;
// the prefix states of the linear-time scan). The logits s_i come from logits.hip.
//
// Work split: one workgroup of 8 waves per (batch, head, 16-column tile of v/o); the d/16 tiles of
// a head are mapped onto one XCD so they share q/k through its L2. The sequence is walked in
// chunks of kC = 64 tokens. After all 8 waves have staged a chunk in LDS, two groups run side by
// side until the end-of-chunk barrier (each SIMD holds one wave of each group):
//   waves 0-3, queries [16w, 16w+16) of the chunk:
//     intra:  A^T = K Q^T (MFMA), W_{t,i} = A (norms folded in) (a_t e^{s_i-m_t} + b_t s_i + g_t)
//             for i <= t, o^T += V^T W^T (MFMA; W stays in registers: its accumulator layout is
//             the B-operand layout up to a permutation of the contraction index, mirrored in V^T);
//     inter:  o_t += q^_t (cX_t X + b_t Y + kappa_t H) with the states at t0 (MFMA), then o.
//   waves 4-7, state rows [(w-4) d/4, (w-3) d/4): X, Y, H advanced to t1 (elementwise rescale,
//     then K^T V' on MFMA), written to the other LDS state buffer; wave 4 also runs the scalar
//     scan of the next chunk.
// States are kept in a centred basis, X = F/E - H/t0 and Y = G - (P/t0) H. Both have zero-sum
// weights, so they stay of the size of the output, and rounding them (and the update operands)
// to bfloat16 for the MFMA is not amplified by the cancellation between alpha F, beta G and
// gamma H. With RoPE, q and k are rotated by their offset inside the chunk and the states are
// kept in the frame of the chunk start, re-based by a fixed rotation after every chunk.
#include <hip/hip_bf16.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace zeros {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kC = 64;          // tokens per chunk
constexpr int kThreads = 512;   // 8 waves: queries 0-3, state rows 4-7
constexpr int kTile = 16;       // value columns per workgroup
constexpr int kPad = 8;         // bf16 elements of row padding in LDS

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    __hip_bfloat162 h = __float22bfloat162_rn(make_float2(lo, hi));
    return *reinterpret_cast<uint32_t *>(&h);
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

template <int D>
struct alignas(16) MSmem {
    alignas(16) uint16_t qh[kC][D + kPad];     // raw (rotated) q rows of the chunk, bf16
    alignas(16) uint16_t kh[kC][D + kPad];     // unit (rotated) k rows, 16-byte blocks swizzled (kswz)
    alignas(16) uint16_t vt[kTile][kC + kPad]; // v tile, transposed: vt[m][token] (also the H update operand)
    alignas(16) uint16_t vx[kTile][kC + kPad]; // update operands v * w_X and v * w_Y (transposed)
    alignas(16) uint16_t vy[kTile][kC + kPad];
    alignas(16) uint16_t st[2][3][kTile][D + kPad];  // X, Y, H transposed, bf16, double-buffered
    float invq[kC];
    Coef cf[2];
};

// Column-block swizzle of the k rows: 16-byte block b of row `key` is stored at b ^ kswz(key),
// so the 8-key column gathers of the state update hit distinct LDS banks.
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

template <int D, bool ROPE>
__global__ __launch_bounds__(kThreads) void causal_mfma_kernel(Problem p, CausalWork work) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    MSmem<D> &sm = *reinterpret_cast<MSmem<D> *>(smem_raw);
    constexpr int NTILE = D / kTile;
    constexpr int KS = D / 32;          // MFMA k-steps over the feature dimension
    constexpr int RT = D / 64;          // 16-row state tiles per update wave
    constexpr int QW = D / 8;           // features per thread in the load phase
    constexpr int NV = QW / 8;          // 16-byte vectors per thread per row slice
    constexpr int NP = QW / 2;          // rotation pairs per thread
    constexpr int kScanWave = 0;        // the query wave with the least intra-chunk work

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const bool qgroup = wave < 4;       // waves 0-3: queries; 4-7: state update
    const int wb = wave & 3;

    const int G = gridDim.x;
    int L = blockIdx.x;
    if ((G & 7) == 0) L = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int tile = L % NTILE;
    const int bh = L / NTILE;
    const int N = p.N;
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint16_t *qg = static_cast<const uint16_t *>(p.q) + row0 * D;
    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + row0 * D;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + row0 * D;
    const uint16_t *g1g = static_cast<const uint16_t *>(p.g1) + row0;
    const uint16_t *ghg = static_cast<const uint16_t *>(p.gh) + row0;
    const float *slog = work.s + row0;
    uint16_t *og = static_cast<uint16_t *>(p.o) + row0 * D;

    // load-phase coordinates: row lr of the chunk, features [f0, f0 + QW), value columns 2*p8+{0,1}
    const int lr = tid >> 3, p8 = tid & 7, f0 = p8 * QW;
    const int sc_lane = tid - 64 * kScanWave;   // lane of the scan wave that loads logits/gates

    // rotation of this thread's pairs by its offset lr inside the chunk
    float rc[ROPE ? NP : 1], rs[ROPE ? NP : 1];
    // rotation re-basing this update lane's state rows by -kC after each chunk
    float fc[ROPE ? 2 * RT : 1], fs[ROPE ? 2 * RT : 1];
    if (ROPE) {
#pragma unroll
        for (int a = 0; a < NP; ++a)
            rope_cos_sin(rope_rev_per_pos(f0 / 2 + a, D, p.rope_base), lr, rc[a], rs[a]);
        if (!qgroup) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const int jp = 8 * (RT * wb + rt) + 2 * g4 + pp;
                    rope_cos_sin(rope_rev_per_pos(jp, D, p.rope_base), kC, fc[2 * rt + pp], fs[2 * rt + pp]);
                }
        }
    }

    f32x4 X[RT], Y[RT], Hm[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[rt][i] = Y[rt][i] = Hm[rt][i] = 0.f;
    float m0 = kNegInf, E0 = 0.f, P0 = 0.f;    // scan carry (kept by the scan wave)

    // prefetch registers
    uint4 pq[NV], pk[NV];
    uint32_t pv;                               // v of token lr, columns 2*p8 (low half) and 2*p8+1
    float ps = 0.f, pg1 = 0.f, pgh = 0.f;     // logits and gates of the chunk after the current one
    auto load_scalars = [&](int tc) {
        if (sc_lane >= 0 && sc_lane < kC) {
            const bool vs = tc + sc_lane < N;
            ps = vs ? slog[tc + sc_lane] : 0.f;
            pg1 = vs ? lo_f(g1g[tc + sc_lane]) : 0.f;
            pgh = vs ? lo_f(ghg[tc + sc_lane]) : 0.f;
        }
    };
    auto load_chunk = [&](int tc) {
        const bool valid = tc + lr < N;
        const size_t base = static_cast<size_t>(tc + lr) * D + f0;
#pragma unroll
        for (int a = 0; a < NV; ++a) {
            pq[a] = valid ? *reinterpret_cast<const uint4 *>(qg + base + 8 * a) : make_uint4(0, 0, 0, 0);
            pk[a] = valid ? *reinterpret_cast<const uint4 *>(kg + base + 8 * a) : make_uint4(0, 0, 0, 0);
        }
        pv = valid ? *reinterpret_cast<const uint32_t *>(vg + static_cast<size_t>(tc + lr) * D + tile * kTile + 2 * p8)
                   : 0u;
    };
    if (N > 0) {
        load_chunk(0);
        load_scalars(0);
        if (wave == kScanWave) chunk_scan(sm.cf[0], lane, 0, min(kC, N), ps, pg1, pgh, m0, E0, P0);
        load_scalars(kC);
    }
    __syncthreads();

    for (int t0 = 0, ci = 0; t0 < N; t0 += kC, ++ci) {
        const int nval = min(kC, N - t0);
        const Coef &cf = sm.cf[ci & 1];

        // ---- registers -> LDS: norms, rotation, v operands, per-key data (all 8 waves)
        {
            float ssq = 0.f, ssk = 0.f;
#pragma unroll
            for (int a = 0; a < NV; ++a) {
                ssq = dot2_bf16(pq[a].x, ssq); ssq = dot2_bf16(pq[a].y, ssq);
                ssq = dot2_bf16(pq[a].z, ssq); ssq = dot2_bf16(pq[a].w, ssq);
                ssk = dot2_bf16(pk[a].x, ssk); ssk = dot2_bf16(pk[a].y, ssk);
                ssk = dot2_bf16(pk[a].z, ssk); ssk = dot2_bf16(pk[a].w, ssk);
            }
            ssq = group_sum<8>(ssq);
            ssk = group_sum<8>(ssk);
            const bool valid = lr < nval;
            const float iq = valid ? __frsqrt_rn(fmaxf(ssq, 1e-24f)) : 0.f;
            const float ik = valid ? __frsqrt_rn(fmaxf(ssk, 1e-24f)) : 0.f;
            if (p8 == 0) sm.invq[lr] = iq;
            // q keeps its norm (1/|q| is applied per query); k is stored as a unit vector
#pragma unroll
            for (int a = 0; a < NV; ++a) {
                uint32_t wq[4] = {pq[a].x, pq[a].y, pq[a].z, pq[a].w};
                uint32_t wk[4] = {pk[a].x, pk[a].y, pk[a].z, pk[a].w};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float k0 = lo_f(wk[b]), k1 = hi_f(wk[b]);
                    if (ROPE) {
                        const float c = rc[4 * a + b], sn = rs[4 * a + b];
                        const float q0 = lo_f(wq[b]), q1 = hi_f(wq[b]);
                        const float ck = c * ik, sk = sn * ik;
                        wq[b] = pack2(q0 * c - q1 * sn, q0 * sn + q1 * c);
                        wk[b] = pack2(k0 * ck - k1 * sk, k0 * sk + k1 * ck);
                    } else {
                        wk[b] = pack2(k0 * ik, k1 * ik);
                    }
                }
                pq[a] = make_uint4(wq[0], wq[1], wq[2], wq[3]);
                pk[a] = make_uint4(wk[0], wk[1], wk[2], wk[3]);
            }
            const int ksw = kswz(lr);
#pragma unroll
            for (int a = 0; a < NV; ++a) {
                const int blk = f0 / 8 + a;
                *reinterpret_cast<uint4 *>(&sm.qh[lr][8 * blk]) = pq[a];
                *reinterpret_cast<uint4 *>(&sm.kh[lr][8 * (blk ^ ksw)]) = pk[a];
            }
            // v operands, stored transposed as token pairs: the lanes of rows 2a and 2a+1 (8 lanes
            // apart, same DPP row) swap their column pairs, then row 2a writes column 2 p8 and
            // row 2a+1 column 2 p8 + 1 for tokens (2a, 2a+1). Weights are zero past the chunk end.
            const uint32_t other = static_cast<uint32_t>(
                __builtin_amdgcn_update_dpp(0, static_cast<int>(pv), kRowRor + 8, 0xf, 0xf, false));
            const bool odd = lr & 1;
            const uint32_t pair = odd ? ((other >> 16) | (pv & 0xffff0000u)) : ((pv & 0xffffu) | (other << 16));
            const int col = 2 * p8 + (odd ? 1 : 0), tok = lr & ~1;
            const float2 wx2 = *reinterpret_cast<const float2 *>(&cf.wx[tok]);
            const float2 wy2 = *reinterpret_cast<const float2 *>(&cf.wy[tok]);
            const float v0 = lo_f(pair), v1 = hi_f(pair);
            *reinterpret_cast<uint32_t *>(&sm.vt[col][tok]) = pair;
            *reinterpret_cast<uint32_t *>(&sm.vx[col][tok]) = pack2(v0 * wx2.x, v1 * wx2.y);
            *reinterpret_cast<uint32_t *>(&sm.vy[col][tok]) = pack2(v0 * wy2.x, v1 * wy2.y);
        }
        lds_barrier();
        if (t0 + kC < N) load_chunk(t0 + kC);
        // ---- coefficients of the next chunk; then fetch the logits and gates of the one after
        if (wave == kScanWave && t0 + kC < N) {
            chunk_scan(sm.cf[(ci + 1) & 1], lane, t0 + kC, min(kC, N - t0 - kC), ps, pg1, pgh, m0, E0, P0);
            load_scalars(t0 + 2 * kC);
        }

        if (qgroup) {
            // ---- A^T tiles for this wave's query block
            const int tb = wb;
            bf16x8 qop[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qop[ks] = *reinterpret_cast<const bf16x8 *>(&sm.qh[16 * tb + l16][32 * ks + 8 * g4]);
            f32x4 at[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) at[kb][i] = 0.f;
                if (kb <= tb) {
                    const int key = 16 * kb + l16;
                    const int ksw = kswz(key);
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sm.kh[key][8 * ((4 * ks + g4) ^ ksw)]);
                        at[kb] = mfma(a, qop[ks], at[kb]);
                    }
                }
            }

            // ---- intra-chunk weights and o^T = V^T W^T
            const int tq = 16 * tb + l16;
            const float iq = sm.invq[tq], qa = cf.qa[tq], qm = cf.qm[tq], qb = cf.qb[tq], qgm = cf.qg[tq];
            const bool exact_exp = cf.chunk[6] != 0.f;   // uniform: logits jumped by > e^60 in the chunk
            f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pi = 0; pi < 2; ++pi) {
                if (2 * pi > tb) continue;
                uint32_t wv[4] = {0u, 0u, 0u, 0u};
                uint2 va[2] = {make_uint2(0, 0), make_uint2(0, 0)};
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
                        const float x = at[kb][i] * iq * (qa * ke_[i] + qb * ks_[i] + qgm);
                        w[i] = (key <= tq && tq < nval) ? x : 0.f;
                    }
                    wv[2 * h2] = pack2(w[0], w[1]);
                    wv[2 * h2 + 1] = pack2(w[2], w[3]);
                    va[h2] = *reinterpret_cast<const uint2 *>(&sm.vt[l16][16 * kb + 4 * g4]);
                }
                oacc = mfma(as_bf16x8(va[0].x, va[0].y, va[1].x, va[1].y), as_bf16x8(wv[0], wv[1], wv[2], wv[3]), oacc);
            }

            // ---- carried states
            if (t0 > 0) {
                const int sb = ci & 1;
                f32x4 ax = {0.f, 0.f, 0.f, 0.f}, ay = ax, ah = ax;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    ax = mfma(*reinterpret_cast<const bf16x8 *>(&sm.st[sb][0][l16][32 * ks + 8 * g4]), qop[ks], ax);
                    ay = mfma(*reinterpret_cast<const bf16x8 *>(&sm.st[sb][1][l16][32 * ks + 8 * g4]), qop[ks], ay);
                    ah = mfma(*reinterpret_cast<const bf16x8 *>(&sm.st[sb][2][l16][32 * ks + 8 * g4]), qop[ks], ah);
                }
                const float cx = cf.qcx[tq], kap = cf.qkap[tq];
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[i] += iq * (cx * ax[i] + qb * ay[i] + kap * ah[i]);
            }
            if (tq < nval) {
                const uint2 ov = make_uint2(pack2(oacc[0], oacc[1]), pack2(oacc[2], oacc[3]));
                *reinterpret_cast<uint2 *>(og + static_cast<size_t>(t0 + tq) * D + tile * kTile + 4 * g4) = ov;
            }
        } else {
            // ---- advance the states to t1
            if (t0 > 0) {
                const float rX = cf.chunk[3], cHX = cf.chunk[4], cHY = cf.chunk[5];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        X[rt][i] = rX * X[rt][i] + cHX * Hm[rt][i];
                        Y[rt][i] = Y[rt][i] + cHY * Hm[rt][i];
                    }
            }
            const int gsw = 2 * g4;             // kswz of every key this lane gathers
#pragma unroll
            for (int ks2 = 0; ks2 < kC / 32; ++ks2) {
                const int kk0 = 32 * ks2 + 8 * g4;
                const bf16x8 BX = *reinterpret_cast<const bf16x8 *>(&sm.vx[l16][kk0]);
                const bf16x8 BY = *reinterpret_cast<const bf16x8 *>(&sm.vy[l16][kk0]);
                const bf16x8 BH = *reinterpret_cast<const bf16x8 *>(&sm.vt[l16][kk0]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const int j = 16 * (RT * wb + rt) + l16;
                    const int jc = (((j >> 3) ^ gsw) << 3) | (j & 7);
                    bf16x8 a;
#pragma unroll
                    for (int c = 0; c < 8; ++c) a[c] = static_cast<short>(sm.kh[kk0 + c][jc]);
                    X[rt] = mfma(a, BX, X[rt]);
                    Y[rt] = mfma(a, BY, Y[rt]);
                    Hm[rt] = mfma(a, BH, Hm[rt]);
                }
            }
            if (ROPE) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const float c = fc[2 * rt + pp], sn = fs[2 * rt + pp];
                        const int i0 = 2 * pp, i1 = i0 + 1;
                        float x0 = X[rt][i0], x1 = X[rt][i1];
                        X[rt][i0] = x0 * c + x1 * sn; X[rt][i1] = x1 * c - x0 * sn;
                        x0 = Y[rt][i0]; x1 = Y[rt][i1];
                        Y[rt][i0] = x0 * c + x1 * sn; Y[rt][i1] = x1 * c - x0 * sn;
                        x0 = Hm[rt][i0]; x1 = Hm[rt][i1];
                        Hm[rt][i0] = x0 * c + x1 * sn; Hm[rt][i1] = x1 * c - x0 * sn;
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
        lds_barrier();            // chunk done: LDS staging, states and coefficients may be replaced
    }

    // ---- final state (update waves): back to F = E (X + H/t), G = Y + (P/t) H, absolute RoPE frame
    if (p.st.F != nullptr) {
        if (N > 0) {
            const Coef &cl = sm.cf[((N + kC - 1) / kC - 1) & 1];
            m0 = cl.chunk[0];
            E0 = cl.chunk[1];
            P0 = cl.chunk[2];
        }
        if (!qgroup) {
            const size_t mat0 = static_cast<size_t>(bh) * D * D;
            const float tf = static_cast<float>(N);
            const int nchunks = (N + kC - 1) / kC;
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
                if (ROPE && N > 0) {
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        const int jp = 8 * (RT * wb + rt) + 2 * g4 + pp;
                        float c, sn;
                        rope_cos_sin(rope_rev_per_pos(jp, D, p.rope_base), nchunks * kC, c, sn);
                        const int i0 = 2 * pp, i1 = i0 + 1;
                        float x0 = F[i0], x1 = F[i1];
                        F[i0] = x0 * c - x1 * sn; F[i1] = x0 * sn + x1 * c;
                        x0 = Gv[i0]; x1 = Gv[i1];
                        Gv[i0] = x0 * c - x1 * sn; Gv[i1] = x0 * sn + x1 * c;
                        x0 = Hv[i0]; x1 = Hv[i1];
                        Hv[i0] = x0 * c - x1 * sn; Hv[i1] = x0 * sn + x1 * c;
                    }
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

template <int D, bool ROPE>
hipError_t launch_one(const Problem &p, const CausalWork &w, hipStream_t stream) {
    const size_t smem = sizeof(MSmem<D>);
    const void *fn = reinterpret_cast<const void *>(&causal_mfma_kernel<D, ROPE>);
    static bool attr_set = false;   // idempotent; a race only repeats the same call
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    const int grid = p.B * p.H * (D / kTile);
    hipLaunchKernelGGL((causal_mfma_kernel<D, ROPE>), dim3(grid), dim3(kThreads), smem, stream, p, w);
    return hipGetLastError();
}

}  // namespace

size_t causal_work_bytes(int B, int H, int N, int du) {
    const size_t a = 256;
    const size_t nseg = (static_cast<size_t>(N) + kLogitSeg - 1) / kLogitSeg;
    const size_t s = (static_cast<size_t>(B) * H * N * 4 + a - 1) / a * a;
    const size_t u = (static_cast<size_t>(B) * H * nseg * du * 4 + a - 1) / a * a;
    return s + u;
}

CausalWork causal_work_carve(void *base, int B, int H, int N, int du) {
    const size_t a = 256;
    const size_t s = (static_cast<size_t>(B) * H * N * 4 + a - 1) / a * a;
    CausalWork w;
    w.s = static_cast<float *>(base);
    w.useg = reinterpret_cast<float *>(static_cast<char *>(base) + s);
    (void)du;
    return w;
}

hipError_t launch_causal_mfma(const Problem &p, const CausalWork &w, hipStream_t stream) {
    hipError_t err = launch_logits(p, w.useg, w.s, stream);
    if (err != hipSuccess) return err;
    if (p.d == 128) return p.rope ? launch_one<128, true>(p, w, stream) : launch_one<128, false>(p, w, stream);
    if (p.d == 64) return p.rope ? launch_one<64, true>(p, w, stream) : launch_one<64, false>(p, w, stream);
    return hipErrorInvalidValue;
}

}  // namespace zeros
