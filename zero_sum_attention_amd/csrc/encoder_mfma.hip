// Encoder (non-causal) ZeroS forward on the matrix cores: bfloat16 q/k/v/u, d in {64, 128}.
//
// Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计 (weights
// and prefix states; every query of an encoder uses the full-sequence sums, t = N) with the logits
// of 偏差 logits 设计 over one global prior-smoothed mean ubar. With t = N for every query,
//   alpha_t F + beta_t G + gamma_t H = sigmah_t X + ((sigma1_t - sigmah_t)/N) Y,
//   X = sum_i (e^{s_i - m}/E - 1/N) k^_i^T v_i,   Y = sum_i (s_i - P/N) k^_i^T v_i,
// two centred d x d states (zero-sum weights, so of the size of the output and safe to round to
// bfloat16 as MFMA operands). The optional zero-order gate of the same section (a first layer may
// keep the uniform term) adds (sigma0_t/N) q^_t H with H = sum_i k^_i^T v_i, a third state
// (the G0 instances).
//
// Sequences that encoder_long_path selects (from kEncoderTileMaxN tokens, or large batches) take the
// token-parallel pipeline of encoder_long.hip instead; this file holds the single-launch variants.
//
// One workgroup of 4 waves per (batch, head, 16-column tile of the value dimension): d/16 workgroups
// per head, each computing its tile's columns of X and Y and of the output.
//   A: column sums of u -> ubar; logits s_i (lanes of a token row reduce their partial dots), each
//      row's (max, sum e^{s - max}, sum s) merged by the lane that ends with its dot, then across
//      the workgroup. Every tile workgroup of a head repeats this phase (u from L2).
//   B: per 64-token step, k^ (unit, optionally RoPE-rotated, all features) and the tile's columns
//      of v w_X and v w_Y staged transposed in LDS; wave w advances feature tiles of X and Y on MFMA.
//   C: X^T, Y^T of the tile through LDS as bf16 A operands; the waves take 16-token blocks in turn:
//      o^T = X^T q^T and Y^T q^T on MFMA, scaled per token by sigmah/|q| and (sigma1 - sigmah)/(N |q|).
#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"
#include "encoder_common.hpp"

namespace zeros {
namespace {

constexpr int kEC = 64;            // tokens per step of the state pass
constexpr int kEShortN = 256;      // longest sequence of the short variant (logits buffer in LDS)
constexpr int kEThreads = 256;     // 4 waves
constexpr int kEPad = 8;           // bf16 elements of row padding in LDS

// Sum over the D/8 consecutive lanes that hold one token row (DPP within a row of 16 lanes).
template <int D>
__device__ __forceinline__ float row_sum(float x) { return group_sum<D / 8>(x); }

// The logits of the sequence stay in LDS (N <= NMAX).
template <int D, bool ROPE, int NMAX, bool G0>
__global__ __launch_bounds__(kEThreads) void encoder_mfma_kernel(Problem p) {
    constexpr int NS = G0 ? 3 : 2;     // states: X, Y (and H)
    constexpr int FT = D / 16;         // 16-row feature tiles of a state
    constexpr int FW = FT / 4;         // feature tiles per wave
    constexpr int KS = D / 32;         // 32-feature steps
    constexpr int LPR = D / 8;         // lanes per token row (8 features, 16 bytes each)
    constexpr int RPP = kEThreads / LPR;   // token rows per pass
    __shared__ float ubar[D];
    __shared__ __align__(16) float colp[RPP][D];          // partial column sums of u, one row per token row of a pass
    __shared__ float sl[NMAX];                      // logits of the sequence (N <= NMAX)
    __shared__ float4 red[kEThreads / 64];
    __shared__ __align__(16) uint16_t kt[D][kEC + kEPad];    // k^ of the chunk, transposed
    __shared__ __align__(16) uint16_t vxt[16][kEC + kEPad];  // this tile's columns of v w_X, transposed
    __shared__ __align__(16) uint16_t vyt[16][kEC + kEPad];  // this tile's columns of v w_Y, transposed
    __shared__ __align__(16) uint16_t vht[G0 ? 16 : 1][kEC + kEPad];  // this tile's columns of v (H)
    __shared__ __align__(16) uint16_t sxy[NS][16][D + kEPad]; // X^T, Y^T (H^T) of this tile (bf16), for phase C
    __shared__ double rev[ROPE ? D / 2 : 1];                 // RoPE turns per position of each pair

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    // workgroup (column tile ct, head bh): with B H a multiple of 8 the tiles of a head run on one XCD
    // (workgroups go to the XCDs in turn) and share its L2 for the q, k, u rows every tile reads
    const int bhn = p.B * p.H;
    const int ct = blockIdx.x / bhn, bh = blockIdx.x % bhn;
    const int h = bh % p.H;
    const int N = p.N;
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint16_t *q = static_cast<const uint16_t *>(p.q) + row0 * D;
    const uint16_t *k = static_cast<const uint16_t *>(p.k) + row0 * D;
    const uint16_t *v = static_cast<const uint16_t *>(p.v) + row0 * D;
    const uint16_t *u = static_cast<const uint16_t *>(p.u) + row0 * D;
    const uint16_t *g1 = static_cast<const uint16_t *>(p.g1) + row0;
    const uint16_t *gh = static_cast<const uint16_t *>(p.gh) + row0;
    const uint16_t *g0 = G0 ? static_cast<const uint16_t *>(p.g0) + row0 : nullptr;
    uint16_t *o = static_cast<uint16_t *>(p.o) + row0 * D;
    const float et = expf(p.tau[h]);
    const int fr = tid % LPR, rr = tid / LPR;       // feature group (8 features) and row of a pass
    if (ROPE && tid < D / 2) rev[tid] = rope_rev_per_pos(tid, D, p.rope_base);   // ordered by the first barrier

    // k rows (all features) and this tile's v columns of a step, read one step ahead. Thread (rr, fr)
    // takes the token pairs (2 rr + 2 RPP jj, +1) of features 8 fr + [0, 8); for v, token pair
    // 2 (tid / 4), +1 and columns 16 ct + 4 (tid & 3) + [0, 4). Pairs of tokens make the transposed
    // LDS writes 32-bit.
    constexpr int JR = kEC / RPP;      // rows per thread (even)
    static_assert(JR % 2 == 0 && 2 * kEC <= kEThreads, "state pass shape");
    const int vtk = 2 * (tid >> 2), vcq = tid & 3;
    const bool vthr = tid < 2 * kEC;   // kEC / 2 token pairs x 4 column quads
    auto krow = [&](const int j) { return 2 * rr + (j & 1) + 2 * RPP * (j >> 1); };
    uint4 kn[JR];
    uint2 vn[2] = {make_uint2(0, 0), make_uint2(0, 0)};
    auto load_kv = [&](const int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < JR; ++j)
            kn[j] = *reinterpret_cast<const uint4 *>(k + static_cast<size_t>(min(t0 + krow(j), N - 1)) * D + 8 * fr);   // zeroed below
        if (vthr) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                vn[e] = *reinterpret_cast<const uint2 *>(v + static_cast<size_t>(min(t0 + vtk + e, N - 1)) * D + 16 * ct + 4 * vcq);
        }
    };
    load_kv(0);                        // the first step's rows are in flight during phase A
    // phase C's first q rows and gates of this wave (token block w), read now so that phase C
    // starts without a memory round trip
    constexpr int KS0 = D / 32;
    uint4 qn[KS0];
    uint32_t g1n = 0, ghn = 0, g0n = 0;
    auto load_q = [&](const int tb) __attribute__((always_inline)) {
        const int t = min(16 * tb + l16, N - 1);   // in bounds; rows past N are never stored
        const size_t tr = static_cast<size_t>(t) * D;
#pragma unroll
        for (int ks = 0; ks < KS0; ++ks) qn[ks] = *reinterpret_cast<const uint4 *>(q + tr + 32 * ks + 8 * g4);
        g1n = g1[t];
        ghn = gh[t];
        if (G0) g0n = g0[t];
    };
    const int ntb = (N + 15) / 16;
    if (w < ntb) load_q(w);

    // ---- A: ubar, logits, and the scalar sums. The first UC rows of each thread are read once and
    // stay in registers from the column sums to the logits.
    constexpr int UC = 8;
    const float mu_t = tid < D ? p.mu[h * D + tid] : 0.f;   // read early: used after the first barrier
    uint4 ur[UC];
#pragma unroll
    for (int j = 0; j < UC; ++j)
        ur[j] = *reinterpret_cast<const uint4 *>(u + static_cast<size_t>(min(rr + RPP * j, N - 1)) * D + 8 * fr);
    {
        float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < UC; ++j) {
            if (rr + RPP * j < N) {
                float x[8];
                unpack8(ur[j], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) cs[i] += x[i];
            }
        }
        for (int r = rr + RPP * UC; r < N; r += RPP) {
            float x[8];
            unpack8(*reinterpret_cast<const uint4 *>(u + static_cast<size_t>(r) * D + 8 * fr), x);
#pragma unroll
            for (int i = 0; i < 8; ++i) cs[i] += x[i];
        }
        // every thread's partial column sums through LDS, then one thread per feature adds the RPP
        // rows in order (no cross-lane shuffles)
        *reinterpret_cast<float4 *>(&colp[rr][8 * fr]) = make_float4(cs[0], cs[1], cs[2], cs[3]);
        *reinterpret_cast<float4 *>(&colp[rr][8 * fr + 4]) = make_float4(cs[4], cs[5], cs[6], cs[7]);
        __syncthreads();
        if (tid < D) {
            float su = 0.f;
#pragma unroll
            for (int g = 0; g < RPP; ++g) su += colp[g][tid];
            ubar[tid] = (et * mu_t + su) / (et + static_cast<float>(N));
        }
        __syncthreads();
    }
    // logits, with each row's (max, sum e^{s - max}, sum s) taken by the lane that ends with its dot
    float mloc = kNegInf, eloc = 0.f, ploc = 0.f;
    {
        float ub[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ub[i] = ubar[8 * fr + i];
        const float rs_du = 1.f / sqrtf(static_cast<float>(D));
        auto row = [&](const uint4 &raw, const int r) __attribute__((always_inline)) {
            float dot = 0.f;
            if (r < N) {
                float x[8];
                unpack8(raw, x);
#pragma unroll
                for (int i = 0; i < 8; ++i) dot = fmaf(x[i], ub[i], dot);
            }
            dot = row_sum<D>(dot);                 // every lane of the row calls this (a shuffle)
            if (r < N && fr == 0) {
                const float sv = -dot * rs_du;
                sl[r] = sv;
                lse_merge(mloc, eloc, sv, 1.f);
                ploc += sv;
            }
        };
#pragma unroll
        for (int j = 0; j < UC; ++j) row(ur[j], rr + RPP * j);
        for (int r0 = RPP * UC; r0 < N; r0 += RPP) {   // uniform trip count
            const int r = r0 + rr;
            row(*reinterpret_cast<const uint4 *>(u + static_cast<size_t>(min(r, N - 1)) * D + 8 * fr), r);
        }
    }
    // block reduction of (max, sum e^{s - max}, sum s): in each wave, then across the waves
    wave_lse_merge(mloc, eloc, ploc);
    if (lane == 0) red[w] = make_float4(mloc, eloc, ploc, 0.f);
    __syncthreads();                           // also orders the logits before phase B
    float M = kNegInf, E = 0.f, P = 0.f;
#pragma unroll
    for (int i = 0; i < kEThreads / 64; ++i) {
        const float4 rv = red[i];
        lse_merge(M, E, rv.x, rv.y);
        P += rv.z;
    }
    const float invN = N > 0 ? 1.f / static_cast<float>(N) : 0.f;
    const float invE = E > 0.f ? 1.f / E : 0.f;
    const float PN = P * invN;

    // ---- B: this tile's columns of X = K^T diag(w_X) V and Y = K^T diag(w_Y) V over chunks of kEC
    // tokens; wave w owns feature tiles [FW w, FW w + FW)
    f32x4 X[FW], Y[FW], Hc[G0 ? FW : 1];
#pragma unroll
    for (int j = 0; j < FW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[j][i] = Y[j][i] = 0.f;
#pragma unroll
    for (int j = 0; j < (G0 ? FW : 1); ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) Hc[j][i] = 0.f;
    for (int t0 = 0; t0 < N; t0 += kEC) {
        uint4 kc[JR];
#pragma unroll
        for (int j = 0; j < JR; ++j) kc[j] = kn[j];
        const uint2 vc0 = vn[0], vc1 = vn[1];
        if (t0 + kEC < N) load_kv(t0 + kEC);
#pragma unroll
        for (int jj = 0; jj < JR / 2; ++jj) {
            float kp[2][8];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = t0 + krow(2 * jj + e);
                const bool ok = r < N;
                float(&kv)[8] = kp[e];
                unpack8(ok ? kc[2 * jj + e] : make_uint4(0, 0, 0, 0), kv);
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = fmaf(kv[i], kv[i], ss);
                ss = row_sum<D>(ss);
                const float ik = ok ? __frsqrt_rn(fmaxf(ss, 1e-24f)) : 0.f;
                if (ROPE) {
#pragma unroll
                    for (int j2 = 0; j2 < 4; ++j2) {
                        float cs, sn;
                        rope_cos_sin(rev[4 * fr + j2], r, cs, sn);
                        const float a = kv[2 * j2], b = kv[2 * j2 + 1];
                        kv[2 * j2] = a * cs - b * sn;
                        kv[2 * j2 + 1] = a * sn + b * cs;
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) kv[i] *= ik;
            }
            const int rl = krow(2 * jj);
#pragma unroll
            for (int i = 0; i < 8; ++i) *reinterpret_cast<uint32_t *>(&kt[8 * fr + i][rl]) = pack2(kp[0][i], kp[1][i]);
        }
        if (vthr) {
            float wx[2], wy[2], wh[2], vv[2][4];
            const uint2 vcs[2] = {vc0, vc1};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = t0 + vtk + e;
                const bool ok = r < N;
                const float s = ok ? sl[r] : 0.f;
                wx[e] = ok ? __expf(s - M) * invE - invN : 0.f;
                wy[e] = ok ? s - PN : 0.f;
                wh[e] = ok ? 1.f : 0.f;             // rows past N read row N-1: zero them for H
                vv[e][0] = lo_f(vcs[e].x);
                vv[e][1] = hi_f(vcs[e].x);
                vv[e][2] = lo_f(vcs[e].y);
                vv[e][3] = hi_f(vcs[e].y);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<uint32_t *>(&vxt[4 * vcq + i][vtk]) = pack2(vv[0][i] * wx[0], vv[1][i] * wx[1]);
                *reinterpret_cast<uint32_t *>(&vyt[4 * vcq + i][vtk]) = pack2(vv[0][i] * wy[0], vv[1][i] * wy[1]);
                if (G0)
                    *reinterpret_cast<uint32_t *>(&vht[4 * vcq + i][vtk]) = pack2(vv[0][i] * wh[0], vv[1][i] * wh[1]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks2 = 0; ks2 < kEC / 32; ++ks2) {
            const int kk0 = 32 * ks2 + 8 * g4;
            const bf16x8 BX = *reinterpret_cast<const bf16x8 *>(&vxt[l16][kk0]);
            const bf16x8 BY = *reinterpret_cast<const bf16x8 *>(&vyt[l16][kk0]);
            const bf16x8 BH = G0 ? *reinterpret_cast<const bf16x8 *>(&vht[l16][kk0]) : BY;
#pragma unroll
            for (int j = 0; j < FW; ++j) {
                const bf16x8 A = *reinterpret_cast<const bf16x8 *>(&kt[16 * (FW * w + j) + l16][kk0]);
                X[j] = mfma(A, BX, X[j]);
                Y[j] = mfma(A, BY, Y[j]);
                if (G0) Hc[j] = mfma(A, BH, Hc[j]);
            }
        }
        __syncthreads();
    }
    // X^T and Y^T of the tile into LDS as bf16: accumulator lane (g4, l16) holds features
    // 16 ft + 4 g4 + [0, 4) of column l16
#pragma unroll
    for (int j = 0; j < FW; ++j) {
        const int f = 16 * (FW * w + j) + 4 * g4;
        *reinterpret_cast<uint2 *>(&sxy[0][l16][f]) = make_uint2(pack2(X[j][0], X[j][1]), pack2(X[j][2], X[j][3]));
        *reinterpret_cast<uint2 *>(&sxy[1][l16][f]) = make_uint2(pack2(Y[j][0], Y[j][1]), pack2(Y[j][2], Y[j][3]));
        if (G0)
            *reinterpret_cast<uint2 *>(&sxy[NS - 1][l16][f]) =
                make_uint2(pack2(Hc[j][0], Hc[j][1]), pack2(Hc[j][2], Hc[j][3]));
    }
    __syncthreads();

    // ---- C: outputs of this tile's columns, 16 tokens per step, the waves taking steps in turn.
    // A operands X^T, Y^T (column l16, features 32 ks + 8 g4 + [0, 8)); B operand q^ of token
    // 16 tb + l16, the same features. The next step's q rows and gates are read while this one computes.
    bf16x8 AX[KS], AY[KS], AH[G0 ? KS : 1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        AX[ks] = *reinterpret_cast<const bf16x8 *>(&sxy[0][l16][32 * ks + 8 * g4]);
        AY[ks] = *reinterpret_cast<const bf16x8 *>(&sxy[1][l16][32 * ks + 8 * g4]);
        if (G0) AH[ks] = *reinterpret_cast<const bf16x8 *>(&sxy[NS - 1][l16][32 * ks + 8 * g4]);
    }
    for (int tb = w; tb < ntb; tb += kEThreads / 64) {
        const int t = 16 * tb + l16;
        const bool ok = t < N;
        uint4 qv[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qv[ks] = qn[ks];
        const uint32_t g1v = g1n, ghv = ghn, g0v = g0n;
        if (tb + kEThreads / 64 < ntb) load_q(tb + kEThreads / 64);
        float ss = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint32_t wv[4] = {qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = dot2_bf16(wv[i], ss);
            if (ROPE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // the pair (2j, 2j+1) sits in one 32-bit word: j = 16 ks + 4 g4 + i
                    float cs, sn;
                    rope_cos_sin(rev[16 * ks + 4 * g4 + i], t, cs, sn);
                    const float a = lo_f(wv[i]), b = hi_f(wv[i]);
                    wv[i] = pack2(a * cs - b * sn, a * sn + b * cs);
                }
                qv[ks] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float iq = ok ? __frsqrt_rn(fmaxf(ss, 1e-24f)) : 0.f;
        const float s1 = ok ? __fdividef(1.f, 1.f + __expf(-lo_f(g1v))) : 0.f;
        const float sh = ok ? __fdividef(1.f, 1.f + __expf(-lo_f(ghv))) : 0.f;
        const float ax = sh * iq, ay = (s1 - sh) * invN * iq;
        const float ah = (G0 && ok) ? __fdividef(1.f, 1.f + __expf(-lo_f(g0v))) * invN * iq : 0.f;
        f32x4 accX = {0.f, 0.f, 0.f, 0.f}, accY = accX, accH = accX;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 B = as_bf16x8(qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w);
            accX = mfma(AX[ks], B, accX);
            accY = mfma(AY[ks], B, accY);
            if (G0) accH = mfma(AH[ks], B, accH);
        }
        if (ok) {
            float r4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r4[i] = ax * accX[i] + ay * accY[i] + (G0 ? ah * accH[i] : 0.f);
            *reinterpret_cast<uint2 *>(o + static_cast<size_t>(t) * D + 16 * ct + 4 * g4) =
                make_uint2(pack2(r4[0], r4[1]), pack2(r4[2], r4[3]));
        }
    }
}

// ---- Per-head variant for short sequences (N <= kEHeadMaxN, d = 64): one workgroup of 16 waves per
// (batch, head) does the u sums, the logits and the unit k^ once for all column tiles (the tile
// variant above repeats them per tile), reads all of u, k, v and the first q block of each wave at
// its start (one memory round trip), stages all tokens at once for the states (128 at a time with
// RoPE), and gives each
// wave its own 16 x 16 tiles of X and Y (and H) and its own 16-token block of outputs.
constexpr int kEHeadMaxN = 256;
constexpr int kEHThreads = 1024;
// tokens staged per round of the state pass: all of them, or 128 with RoPE (whose angle arithmetic
// for two rows at once would spill)
constexpr int kEHalf = 256;
template <bool ROPE> constexpr int eh_round() { return ROPE ? 128 : kEHalf; }

template <int D, bool G0>
union EHeadBuf {
    float colp[kEHThreads / 16][D];                  // partial column sums of u, one per 16-lane row
    struct {
        uint16_t kt[D][kEHalf + kEPad];             // k^ of the round, transposed
        uint16_t vxt[D][kEHalf + kEPad];            // v w_X of the round, transposed
        uint16_t vyt[D][kEHalf + kEPad];            // v w_Y
        uint16_t vht[G0 ? D : 1][kEHalf + kEPad];   // v (the H state of the zero-order gate)
    } st;
    uint16_t sxy[G0 ? 3 : 2][D][D + kEPad];         // X^T, Y^T (H^T) as bf16, for the outputs
};

template <int D, bool ROPE, bool G0>
__global__ __launch_bounds__(kEHThreads) void encoder_head_kernel(Problem p) {
    constexpr int NS = G0 ? 3 : 2;
    constexpr int LPR = D / 8;                   // lanes per token row (8 features each)
    constexpr int RPP = kEHThreads / LPR;        // token rows per pass
    constexpr int UP = kEHeadMaxN / RPP;         // passes (rows per thread)
    constexpr int ER = eh_round<ROPE>();         // tokens per staging round
    constexpr int JPH = ER / RPP;                // passes per staging round
    constexpr int NFT = D / 16;                  // 16-row (16-column) tiles of a d x d state
    // waves that form the states and the block of BF x BC 16 x 16 tiles each one owns: without RoPE
    // eight waves of 1 x 2 tiles (each k^ operand read from LDS serves two tiles; sixteen waves of
    // one tile read every operand four times over), with RoPE (fewer free registers) sixteen
    static_assert(D == 64, "per-head variant: d = 64");
    constexpr int PBW = ROPE ? 16 : 8;
    constexpr int BF = 1, BC = ROPE ? 1 : 2;
    constexpr int TPW = BF * BC;                 // state tiles per wave
    static_assert(PBW * TPW == NFT * NFT, "state tiles");
    constexpr int KS = D / 32;                   // 32-feature steps of the output products
    static_assert(UP * RPP == kEHeadMaxN && JPH * RPP == ER && TPW >= 1, "per-head shape");
    __shared__ __align__(16) EHeadBuf<D, G0> buf;
    __shared__ float ubar[D];
    __shared__ float sl[kEHeadMaxN];
    __shared__ float4 red[16];
    __shared__ float red2[16];
    __shared__ double rev[ROPE ? D / 2 : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int bh = blockIdx.x, h = bh % p.H;
    const int N = p.N;
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint16_t *q = static_cast<const uint16_t *>(p.q) + row0 * D;
    const uint16_t *k = static_cast<const uint16_t *>(p.k) + row0 * D;
    const uint16_t *v = static_cast<const uint16_t *>(p.v) + row0 * D;
    const uint16_t *u = static_cast<const uint16_t *>(p.u) + row0 * D;
    const uint16_t *g1 = static_cast<const uint16_t *>(p.g1) + row0;
    const uint16_t *gh = static_cast<const uint16_t *>(p.gh) + row0;
    const uint16_t *g0 = G0 ? static_cast<const uint16_t *>(p.g0) + row0 : nullptr;
    uint16_t *o = static_cast<uint16_t *>(p.o) + row0 * D;
    const int fr = tid % LPR, rr = tid / LPR;    // feature group and row of a pass
    if (ROPE && tid < D / 2) rev[tid] = rope_rev_per_pos(tid, D, p.rope_base);   // ordered by the first barrier

    // ---- every read up front: rows rr + RPP j of u, k, v (clamped into the sequence; rows past N
    // are zeroed where used), and this wave's 16-token block of q with its gates
    uint4 ur[UP], kr[UP], vr[UP];
#pragma unroll
    for (int j = 0; j < UP; ++j)       // u first: phase A waits for these only
        ur[j] = *reinterpret_cast<const uint4 *>(u + static_cast<size_t>(min(rr + RPP * j, N - 1)) * D + 8 * fr);
#pragma unroll
    for (int j = 0; j < UP; ++j) {
        const size_t off = static_cast<size_t>(min(rr + RPP * j, N - 1)) * D + 8 * fr;
        kr[j] = *reinterpret_cast<const uint4 *>(k + off);
        vr[j] = *reinterpret_cast<const uint4 *>(v + off);
    }
    // (the RoPE variant with the zero-order gate reads them at phase C: its registers are full)
    constexpr bool EARLY_Q = !(ROPE && G0);
    const int tq = min(16 * w + l16, N - 1);
    uint4 qv[KS];
    uint32_t g1v = 0, ghv = 0, g0v = 0;
    auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qv[ks] = *reinterpret_cast<const uint4 *>(q + static_cast<size_t>(tq) * D + 32 * ks + 8 * g4);
        g1v = g1[tq];
        ghv = gh[tq];
        if (G0) g0v = g0[tq];
    };
    if (EARLY_Q) load_q();
    const float et = expf(p.tau[h]);
    const float mu_t = tid < 4 * D ? p.mu[h * D + (tid >> 2)] : 0.f;

    // ---- A: ubar = (e^tau mu + sum u) / (e^tau + N). Per thread the column sums of its rows; for
    // d = 64 the two token rows of a 16-lane row are added by DPP (row_ror 8); one partial per
    // 16-lane row goes to LDS, and 4 d threads add them (16 each, then the 4 by DPP).
    {
        float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < UP; ++j) {
            float x[8];
            unpack8(ur[j], x);
            const bool ok = rr + RPP * j < N;
#pragma unroll
            for (int i = 0; i < 8; ++i) cs[i] += ok ? x[i] : 0.f;
        }
        if constexpr (LPR == 8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) cs[i] += dpp_mov<kRowRor + 8>(cs[i]);
        }
        if ((lane & 15) < LPR) {
            float *dst = &buf.colp[tid >> 4][8 * fr];
            *reinterpret_cast<float4 *>(dst) = make_float4(cs[0], cs[1], cs[2], cs[3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(cs[4], cs[5], cs[6], cs[7]);
        }
        __syncthreads();
        if (tid < 4 * D) {
            const int f = tid >> 2, qq = tid & 3;
            float su = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) su += buf.colp[16 * qq + e][f];
            su = group_sum<4>(su);
            if (qq == 0) ubar[f] = (et * mu_t + su) / (et + static_cast<float>(N));
        }
        __syncthreads();
    }
    // logits s_r = -(u_r . ubar) / sqrt(d) and their (max, sum e^{s - max}, sum s): the maximum
    // first (wave DPP max, then the 16 waves through LDS), then one exponential per row
    float mx = kNegInf, ps = 0.f;
    {
        float ub[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ub[i] = ubar[8 * fr + i];
        const float rs_du = 1.f / sqrtf(static_cast<float>(D));
#pragma unroll
        for (int j = 0; j < UP; ++j) {
            const int r = rr + RPP * j;
            float x[8];
            unpack8(ur[j], x);
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) dot = fmaf(x[i], ub[i], dot);
            dot = group_sum<LPR>(dot);
            if (r < N && fr == 0) {
                const float sv = -dot * rs_du;
                sl[r] = sv;
                mx = fmaxf(mx, sv);
                ps += sv;
            }
        }
    }
    mx = lane_f(wave_scan_max(mx), 63);
    ps = lane_f(wave_scan_add(ps), 63);
    if (lane == 0) red[w] = make_float4(mx, ps, 0.f, 0.f);
    __syncthreads();
    float M = kNegInf, P = 0.f;
    {
        const float4 rv = red[l16];
        float m = rv.x, q4 = rv.y;
        m = fmaxf(m, dpp_mov<kQuadXor1>(m));
        q4 += dpp_mov<kQuadXor1>(q4);
        m = fmaxf(m, dpp_mov<kQuadXor2>(m));
        q4 += dpp_mov<kQuadXor2>(q4);
        m = fmaxf(m, dpp_mov<kRowHalfMirror>(m));
        q4 += dpp_mov<kRowHalfMirror>(q4);
        m = fmaxf(m, dpp_mov<kRowMirror>(m));
        q4 += dpp_mov<kRowMirror>(q4);
        M = lane_f(m, 0);
        P = lane_f(q4, 0);
    }
    float es = 0.f;
#pragma unroll
    for (int j = 0; j < UP; ++j) {   // each lane reads back only the logits it wrote
        const int r = rr + RPP * j;
        if (r < N && fr == 0) es += __expf(sl[r] - M);
    }
    es = lane_f(wave_scan_add(es), 63);
    if (lane == 0) red2[w] = es;
    __syncthreads();                               // also orders sl before the state pass
    float E;
    {
        float e4 = red2[l16];
        e4 += dpp_mov<kQuadXor1>(e4);
        e4 += dpp_mov<kQuadXor2>(e4);
        e4 += dpp_mov<kRowHalfMirror>(e4);
        e4 += dpp_mov<kRowMirror>(e4);
        E = lane_f(e4, 0);
    }
    const float invN = 1.f / static_cast<float>(N);
    const float invE = E > 0.f ? 1.f / E : 0.f;
    const float PN = P * invN;

    // ---- B: X = K^T diag(w_X) V, Y = K^T diag(w_Y) V (H = K^T V), ER tokens per round; wave w < PBW
    // owns the feature tiles ftb + [0, BF) x column tiles ctb + [0, BC) of every state
    const int ftb = (w / (NFT / BC)) * BF, ctb = (w % (NFT / BC)) * BC;   // this wave's first tiles (w < PBW)
    f32x4 X[TPW], Y[TPW], Hc[G0 ? TPW : 1];
#pragma unroll
    for (int i = 0; i < TPW; ++i) X[i] = Y[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < (G0 ? TPW : 1); ++i) Hc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nrounds = (N + ER - 1) / ER;
    for (int rd = 0; rd < nrounds; ++rd) {
#pragma unroll
        for (int j = 0; j < UP; ++j) {
            if (j / JPH != rd) continue;           // uniform: this pass's rows belong to the round
            const int r = rr + RPP * j, rl = r - ER * rd;
            const bool ok = r < N;
            float kv[8], vv[8];
            unpack8(kr[j], kv);
            unpack8(vr[j], vv);
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(kv[i], kv[i], ss);
            ss = group_sum<LPR>(ss);
            const float ik = ok ? __frsqrt_rn(fmaxf(ss, 1e-24f)) : 0.f;
            if (ROPE) {
#pragma unroll
                for (int j2 = 0; j2 < 4; ++j2) {
                    float cs, sn;
                    rope_cos_sin(rev[4 * fr + j2], r, cs, sn);
                    const float a = kv[2 * j2], b = kv[2 * j2 + 1];
                    kv[2 * j2] = a * cs - b * sn;
                    kv[2 * j2 + 1] = a * sn + b * cs;
                }
            }
            const float sv = ok ? sl[r] : 0.f;
            const float wx = ok ? __expf(sv - M) * invE - invN : 0.f;
            const float wy = ok ? sv - PN : 0.f;
            const float wh = ok ? 1.f : 0.f;
            const int cl = eh_col(8 * fr, rl);    // the same for the 8 rows 8 fr + i
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                buf.st.kt[8 * fr + i][cl] = bf16_bits(kv[i] * ik);
                buf.st.vxt[8 * fr + i][cl] = bf16_bits(vv[i] * wx);
                buf.st.vyt[8 * fr + i][cl] = bf16_bits(vv[i] * wy);
                if (G0) buf.st.vht[8 * fr + i][cl] = bf16_bits(vv[i] * wh);
            }
        }
        __syncthreads();
        if (w < PBW) {
#pragma unroll
            for (int ks = 0; ks < ER / 32; ++ks) {
                if (ER * rd + 32 * ks >= N) break;        // steps past the sequence hold zeros only
                const int kk0 = 32 * ks + 8 * g4;
                bf16x8 A[BF], BX[BC], BY[BC], BH[G0 ? BC : 1];
#pragma unroll
                for (int i = 0; i < BF; ++i) {
                    const int fa = 16 * (ftb + i) + l16;
                    A[i] = *reinterpret_cast<const bf16x8 *>(&buf.st.kt[fa][eh_col(fa, kk0)]);
                }
#pragma unroll
                for (int j = 0; j < BC; ++j) {
                    const int fb = 16 * (ctb + j) + l16;
                    BX[j] = *reinterpret_cast<const bf16x8 *>(&buf.st.vxt[fb][eh_col(fb, kk0)]);
                    BY[j] = *reinterpret_cast<const bf16x8 *>(&buf.st.vyt[fb][eh_col(fb, kk0)]);
                    if (G0) BH[j] = *reinterpret_cast<const bf16x8 *>(&buf.st.vht[fb][eh_col(fb, kk0)]);
                }
#pragma unroll
                for (int i = 0; i < BF; ++i)
#pragma unroll
                    for (int j = 0; j < BC; ++j) {
                        X[i * BC + j] = mfma(A[i], BX[j], X[i * BC + j]);
                        Y[i * BC + j] = mfma(A[i], BY[j], Y[i * BC + j]);
                        if (G0) Hc[i * BC + j] = mfma(A[i], BH[j], Hc[i * BC + j]);
                    }
            }
        }
        __syncthreads();
    }
    // X^T, Y^T (H^T) as bf16 A operands: accumulator lane (l16, g4) holds features 16 ft + 4 g4 + [0, 4)
    // of column 16 ct + l16
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
        if (w >= PBW) break;
        const int f = 16 * (ftb + ti / BC) + 4 * g4, c = 16 * (ctb + ti % BC) + l16;
        *reinterpret_cast<uint2 *>(&buf.sxy[0][c][f]) = make_uint2(pack2(X[ti][0], X[ti][1]), pack2(X[ti][2], X[ti][3]));
        *reinterpret_cast<uint2 *>(&buf.sxy[1][c][f]) = make_uint2(pack2(Y[ti][0], Y[ti][1]), pack2(Y[ti][2], Y[ti][3]));
        if (G0)
            *reinterpret_cast<uint2 *>(&buf.sxy[NS - 1][c][f]) =
                make_uint2(pack2(Hc[ti][0], Hc[ti][1]), pack2(Hc[ti][2], Hc[ti][3]));
    }
    __syncthreads();

    // ---- C: wave w forms the outputs of tokens 16 w + [0, 16), all column tiles:
    // o_t = sigmah_t q^_t X + ((sigma1_t - sigmah_t)/N) q^_t Y (+ (sigma0_t/N) q^_t H)
    if (16 * w >= N) return;
    if (!EARLY_Q) load_q();
    const int t = 16 * w + l16;
    const bool ok = t < N;
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint32_t wv[4] = {qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = dot2_bf16(wv[i], ss);
        if (ROPE) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the pair (2j, 2j+1) sits in one 32-bit word: j = 16 ks + 4 g4 + i
                float cs, sn;
                rope_cos_sin(rev[16 * ks + 4 * g4 + i], t, cs, sn);
                const float a = lo_f(wv[i]), b = hi_f(wv[i]);
                wv[i] = pack2(a * cs - b * sn, a * sn + b * cs);
            }
            qv[ks] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float iq = ok ? __frsqrt_rn(fmaxf(ss, 1e-24f)) : 0.f;
    const float s1 = ok ? __fdividef(1.f, 1.f + __expf(-lo_f(g1v))) : 0.f;
    const float sh = ok ? __fdividef(1.f, 1.f + __expf(-lo_f(ghv))) : 0.f;
    const float ax = sh * iq, ay = (s1 - sh) * invN * iq;
    const float ah = (G0 && ok) ? __fdividef(1.f, 1.f + __expf(-lo_f(g0v))) * invN * iq : 0.f;
#pragma unroll
    for (int ct = 0; ct < NFT; ++ct) {
        f32x4 accX = {0.f, 0.f, 0.f, 0.f}, accY = accX, accH = accX;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 B = as_bf16x8(qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w);
            const int f0 = 32 * ks + 8 * g4;
            accX = mfma(*reinterpret_cast<const bf16x8 *>(&buf.sxy[0][16 * ct + l16][f0]), B, accX);
            accY = mfma(*reinterpret_cast<const bf16x8 *>(&buf.sxy[1][16 * ct + l16][f0]), B, accY);
            if (G0) accH = mfma(*reinterpret_cast<const bf16x8 *>(&buf.sxy[NS - 1][16 * ct + l16][f0]), B, accH);
        }
        if (ok) {
            float r4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r4[i] = ax * accX[i] + ay * accY[i] + (G0 ? ah * accH[i] : 0.f);
            *reinterpret_cast<uint2 *>(o + static_cast<size_t>(t) * D + 16 * ct + 4 * g4) =
                make_uint2(pack2(r4[0], r4[1]), pack2(r4[2], r4[3]));
        }
    }
}

template <int D, bool ROPE, bool G0>
hipError_t launch_g(const Problem &p, hipStream_t stream) {
    const dim3 grid((D / 16) * p.B * p.H);
    // short sequences at d = 64: the per-head variant (N >= 1: the front end returns before a launch
    // for N = 0). At d = 128 it would need more than the 128 registers a wave has at 16 waves per CU.
    if constexpr (D == 64) {
        if (p.N <= kEHeadMaxN) {
            hipLaunchKernelGGL((encoder_head_kernel<D, ROPE, G0>), dim3(p.B * p.H), dim3(kEHThreads), 0, stream, p);
            return hipGetLastError();
        }
    }
    if (p.N <= kEShortN) {
        hipLaunchKernelGGL((encoder_mfma_kernel<D, ROPE, kEShortN, G0>), grid, dim3(kEThreads), 0, stream, p);
        return hipGetLastError();
    }
    // (longer sequences take encoder_long.hip: encoder_long_path)
    if (p.N >= kEncoderTileMaxN) return hipErrorInvalidValue;
    hipLaunchKernelGGL((encoder_mfma_kernel<D, ROPE, kEncoderTileMaxN, G0>), grid, dim3(kEThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool ROPE>
hipError_t launch_one(const Problem &p, hipStream_t stream) {
    return p.g0 != nullptr ? launch_g<D, ROPE, true>(p, stream) : launch_g<D, ROPE, false>(p, stream);
}

}  // namespace

hipError_t launch_encoder_mfma(const Problem &p, hipStream_t stream) {
    if (p.d == 128) return p.rope ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    if (p.d == 64) return p.rope ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace zeros
