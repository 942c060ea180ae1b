// Encoder (non-causal) ZeroS forward on the matrix cores: bfloat16 q/k/v/u, d in {64, 128}.
//
// Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计 (weights
// and prefix states; every query of an encoder uses the full-sequence sums, t = N) with the logits
// of 偏差 logits 设计 over one global prior-smoothed mean ubar. With t = N for every query,
//   alpha_t F + beta_t G + gamma_t H = sigmah_t X + ((sigma1_t - sigmah_t)/N) Y,
//   X = sum_i (e^{s_i - m}/E - 1/N) k^_i^T v_i,   Y = sum_i (s_i - P/N) k^_i^T v_i,
// two centred d x d states (zero-sum weights, so of the size of the output and safe to round to
// bfloat16 as MFMA operands).
//
// One workgroup of 4 waves per (batch, head); wave w owns value columns [16 CT w, 16 CT (w+1)) of X
// and Y, all d rows, in float32 registers.
//   A: column sums of u -> ubar; logits s_i (lanes of a token row reduce their partial dots);
//      m = max s, E = sum e^{s-m}, P = sum s by block reductions.
//   B: per 64-token chunk, k^ (unit, optionally RoPE-rotated), v w_X and v w_Y staged transposed in
//      LDS; X += K^T (w_X V), Y += K^T (w_Y V) on MFMA.
//   C: per 16-token block, o^T = X^T q^T and Y^T q^T on MFMA with X^T, Y^T straight from the
//      registers (their row order, {4g + i, 16 + 4g + i} per 32 features, is the order q^ is
//      loaded in), scaled per token by sigmah/|q| and (sigma1 - sigmah)/(N |q|).
#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace zeros {
namespace {

constexpr int kEC = 64;            // tokens per chunk of the state pass
constexpr int kEThreads = 256;     // 4 waves
constexpr int kEPad = 8;           // bf16 elements of row padding in LDS

template <int D>
__device__ __forceinline__ float row_sum(float x) {
    // sum over the D/8 consecutive lanes that hold one token row
#pragma unroll
    for (int off = 1; off < D / 8; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Block-wide max and sum over 256 threads (every thread gets the result).
__device__ __forceinline__ float block_max(float x, float *scratch) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
    __syncthreads();
    return fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
}
__device__ __forceinline__ float block_sum(float x, float *scratch) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
    __syncthreads();
    return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}

__device__ __forceinline__ void unpack8(const uint4 &x, float (&f)[8]) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo_f(w[i]);
        f[2 * i + 1] = hi_f(w[i]);
    }
}

template <int D, bool ROPE>
__global__ __launch_bounds__(kEThreads) void encoder_mfma_kernel(Problem p) {
    constexpr int CT = D / 64;         // 16-column tiles per wave
    constexpr int FT = D / 16;         // 16-row feature tiles
    constexpr int KS = D / 32;         // 32-feature steps
    constexpr int LPR = D / 8;         // lanes per token row (8 features, 16 bytes each)
    constexpr int RPP = kEThreads / LPR;   // token rows per pass
    __shared__ float ubar[D];
    __shared__ float part[RPP][D + 1];
    __shared__ float sl[kEncoderMfmaMaxN];
    __shared__ float red[4];
    __shared__ __align__(16) uint16_t kt[D][kEC + kEPad];    // k^ of the chunk, transposed
    __shared__ __align__(16) uint16_t vxt[D][kEC + kEPad];   // v w_X, transposed
    __shared__ __align__(16) uint16_t vyt[D][kEC + kEPad];   // v w_Y, transposed

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int bh = blockIdx.x;
    const int h = bh % p.H;
    const int N = p.N;
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint16_t *q = static_cast<const uint16_t *>(p.q) + row0 * D;
    const uint16_t *k = static_cast<const uint16_t *>(p.k) + row0 * D;
    const uint16_t *v = static_cast<const uint16_t *>(p.v) + row0 * D;
    const uint16_t *u = static_cast<const uint16_t *>(p.u) + row0 * D;
    const uint16_t *g1 = static_cast<const uint16_t *>(p.g1) + row0;
    const uint16_t *gh = static_cast<const uint16_t *>(p.gh) + row0;
    uint16_t *o = static_cast<uint16_t *>(p.o) + row0 * D;
    const float et = expf(p.tau[h]);
    const int fr = tid % LPR, rr = tid / LPR;       // feature group (8 features) and row of a pass

    // ---- A: ubar, logits, and the scalar sums
    {
        float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int r = rr; r < N; r += RPP) {
            float x[8];
            unpack8(*reinterpret_cast<const uint4 *>(u + static_cast<size_t>(r) * D + 8 * fr), x);
#pragma unroll
            for (int i = 0; i < 8; ++i) cs[i] += x[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) part[rr][8 * fr + i] = cs[i];
        __syncthreads();
        if (tid < D) {
            float su = 0.f;
            for (int g = 0; g < RPP; ++g) su += part[g][tid];
            ubar[tid] = (et * p.mu[h * D + tid] + su) / (et + static_cast<float>(N));
        }
        __syncthreads();
    }
    {
        float ub[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ub[i] = ubar[8 * fr + i];
        const float rs_du = 1.f / sqrtf(static_cast<float>(D));
        for (int r0 = 0; r0 < N; r0 += RPP) {          // uniform trip count: the row reduction is a shuffle
            const int r = r0 + rr;
            float dot = 0.f;
            if (r < N) {
                float x[8];
                unpack8(*reinterpret_cast<const uint4 *>(u + static_cast<size_t>(r) * D + 8 * fr), x);
#pragma unroll
                for (int i = 0; i < 8; ++i) dot = fmaf(x[i], ub[i], dot);
            }
            dot = row_sum<D>(dot);
            if (r < N && fr == 0) sl[r] = -dot * rs_du;
        }
    }
    __syncthreads();
    float mloc = kNegInf;
    for (int r = tid; r < N; r += kEThreads) mloc = fmaxf(mloc, sl[r]);
    const float M = block_max(mloc, red);
    float eloc = 0.f, ploc = 0.f;
    for (int r = tid; r < N; r += kEThreads) {
        eloc += __expf(sl[r] - M);
        ploc += sl[r];
    }
    const float E = block_sum(eloc, red);
    const float P = block_sum(ploc, red);
    const float invN = N > 0 ? 1.f / static_cast<float>(N) : 0.f;
    const float invE = E > 0.f ? 1.f / E : 0.f;
    const float PN = P * invN;

    // ---- B: X = K^T diag(w_X) V, Y = K^T diag(w_Y) V over chunks of kEC tokens
    f32x4 X[FT][CT], Y[FT][CT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) X[ft][ct][i] = Y[ft][ct][i] = 0.f;
    // k and v rows of a chunk, read one chunk ahead
    constexpr int JR = kEC / RPP;
    uint4 kn[JR], vn[JR];
    auto load_kv = [&](const int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < JR; ++j) {
            const int r = t0 + rr + RPP * j;
            const size_t ri = static_cast<size_t>(min(r, N - 1)) * D + 8 * fr;   // in bounds; zeroed below
            kn[j] = *reinterpret_cast<const uint4 *>(k + ri);
            vn[j] = *reinterpret_cast<const uint4 *>(v + ri);
        }
    };
    if (N > 0) load_kv(0);
    for (int t0 = 0; t0 < N; t0 += kEC) {
        uint4 kc[JR], vc[JR];
#pragma unroll
        for (int j = 0; j < JR; ++j) {
            kc[j] = kn[j];
            vc[j] = vn[j];
        }
        if (t0 + kEC < N) load_kv(t0 + kEC);
#pragma unroll
        for (int j = 0; j < JR; ++j) {
            const int rl = rr + RPP * j, r = t0 + rl;
            const bool ok = r < N;
            float kv[8], vv[8];
            unpack8(ok ? kc[j] : make_uint4(0, 0, 0, 0), kv);
            unpack8(ok ? vc[j] : make_uint4(0, 0, 0, 0), vv);
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(kv[i], kv[i], ss);
            ss = row_sum<D>(ss);
            const float ik = ok ? __frsqrt_rn(fmaxf(ss, 1e-24f)) : 0.f;
            if (ROPE) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float cs, sn;
                    rope_cos_sin(rope_rev_per_pos(4 * fr + jj, D, p.rope_base), r, cs, sn);
                    const float a = kv[2 * jj], b = kv[2 * jj + 1];
                    kv[2 * jj] = a * cs - b * sn;
                    kv[2 * jj + 1] = a * sn + b * cs;
                }
            }
            const float s = ok ? sl[r] : 0.f;
            const float wx = ok ? __expf(s - M) * invE - invN : 0.f;
            const float wy = ok ? s - PN : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int f = 8 * fr + i;
                kt[f][rl] = static_cast<uint16_t>(pack2(kv[i] * ik, 0.f) & 0xffffu);
                vxt[f][rl] = static_cast<uint16_t>(pack2(vv[i] * wx, 0.f) & 0xffffu);
                vyt[f][rl] = static_cast<uint16_t>(pack2(vv[i] * wy, 0.f) & 0xffffu);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks2 = 0; ks2 < kEC / 32; ++ks2) {
            const int kk0 = 32 * ks2 + 8 * g4;
            bf16x8 BX[CT], BY[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int c = 16 * (CT * w + ct) + l16;
                BX[ct] = *reinterpret_cast<const bf16x8 *>(&vxt[c][kk0]);
                BY[ct] = *reinterpret_cast<const bf16x8 *>(&vyt[c][kk0]);
            }
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
                const bf16x8 A = *reinterpret_cast<const bf16x8 *>(&kt[16 * ft + l16][kk0]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    X[ft][ct] = mfma(A, BX[ct], X[ft][ct]);
                    Y[ft][ct] = mfma(A, BY[ct], Y[ft][ct]);
                }
            }
        }
        __syncthreads();
    }

    // ---- C: outputs, 16 tokens per step; each wave writes its own columns. The q rows and gates
    // of the next step are read while this one computes.
    uint2 qan[KS], qcn[KS];            // features 32ks + 4g4 + [0,4) and 32ks + 16 + 4g4 + [0,4)
    uint32_t g1n = 0, ghn = 0;
    auto load_q = [&](const int tb) __attribute__((always_inline)) {
        const int t = min(16 * tb + l16, N - 1);   // in bounds; rows past N are never stored
        const size_t tr = static_cast<size_t>(t) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qan[ks] = *reinterpret_cast<const uint2 *>(q + tr + 32 * ks + 4 * g4);
            qcn[ks] = *reinterpret_cast<const uint2 *>(q + tr + 32 * ks + 16 + 4 * g4);
        }
        g1n = g1[t];
        ghn = gh[t];
    };
    const int ntb = (N + 15) / 16;
    if (N > 0) load_q(0);
    for (int tb = 0; tb < ntb; ++tb) {
        const int t = 16 * tb + l16;
        const bool ok = t < N;
        uint2 qa[KS], qc[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qa[ks] = qan[ks];
            qc[ks] = qcn[ks];
        }
        const uint32_t g1v = g1n, ghv = ghn;
        if (tb + 1 < ntb) load_q(tb + 1);
        float ss = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint32_t wv[4] = {qa[ks].x, qa[ks].y, qc[ks].x, qc[ks].y};
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = dot2_bf16(wv[i], ss);
            if (ROPE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // the pair (2j, 2j+1) sits in one 32-bit word
                    const int f0 = 32 * ks + (i < 2 ? 4 * g4 + 2 * i : 16 + 4 * g4 + 2 * (i - 2));
                    float cs, sn;
                    rope_cos_sin(rope_rev_per_pos(f0 / 2, D, p.rope_base), t, cs, sn);
                    const float a = lo_f(wv[i]), b = hi_f(wv[i]);
                    wv[i] = pack2(a * cs - b * sn, a * sn + b * cs);
                }
                qa[ks] = make_uint2(wv[0], wv[1]);
                qc[ks] = make_uint2(wv[2], wv[3]);
            }
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float iq = ok ? __frsqrt_rn(fmaxf(ss, 1e-24f)) : 0.f;
        const float s1 = ok ? __fdividef(1.f, 1.f + __expf(-lo_f(g1v))) : 0.f;
        const float sh = ok ? __fdividef(1.f, 1.f + __expf(-lo_f(ghv))) : 0.f;
        const float ax = sh * iq, ay = (s1 - sh) * invN * iq;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x4 accX = {0.f, 0.f, 0.f, 0.f}, accY = accX;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const f32x4 &x0 = X[2 * ks][ct], &x1 = X[2 * ks + 1][ct];
                const f32x4 &y0 = Y[2 * ks][ct], &y1 = Y[2 * ks + 1][ct];
                const bf16x8 AX = as_bf16x8(pack2(x0[0], x0[1]), pack2(x0[2], x0[3]), pack2(x1[0], x1[1]), pack2(x1[2], x1[3]));
                const bf16x8 AY = as_bf16x8(pack2(y0[0], y0[1]), pack2(y0[2], y0[3]), pack2(y1[0], y1[1]), pack2(y1[2], y1[3]));
                const bf16x8 B = as_bf16x8(qa[ks].x, qa[ks].y, qc[ks].x, qc[ks].y);
                accX = mfma(AX, B, accX);
                accY = mfma(AY, B, accY);
            }
            if (ok) {
                float r4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) r4[i] = ax * accX[i] + ay * accY[i];
                *reinterpret_cast<uint2 *>(o + static_cast<size_t>(t) * D + 16 * (CT * w + ct) + 4 * g4) =
                    make_uint2(pack2(r4[0], r4[1]), pack2(r4[2], r4[3]));
            }
        }
    }
}

template <int D, bool ROPE>
hipError_t launch_one(const Problem &p, hipStream_t stream) {
    hipLaunchKernelGGL((encoder_mfma_kernel<D, ROPE>), dim3(p.B * p.H), dim3(kEThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encoder_mfma(const Problem &p, hipStream_t stream) {
    if (p.d == 128) return p.rope ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    if (p.d == 64) return p.rope ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace zeros
