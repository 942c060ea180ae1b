// Encoder (non-causal) ZeroS forward, float32 VALU path.
//
// Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers": 关键设计 gives
// the weights and the prefix states; 损失函数 / 训练策略 states that the encoder mode exists. With
// every query using the full-sequence sums (t = N) and one global prior-smoothed mean ubar,
//   alpha_t F + beta_t G + gamma_t H = sigmah_t X + ((sigma1_t - sigmah_t)/N) Y,
//   X = sum_i (e^{s_i}/E - 1/N) k^_i^T v_i = F/E - H/N,   Y = sum_i (s_i - P/N) k^_i^T v_i = G - (P/N) H,
// so two centred d x d states carry the whole output. The optional zero-order gate (same section:
// a first layer may keep the uniform term) adds (sigma0_t / N) q^_t H.
//
// One workgroup per (batch, head, 16-column tile). Pass 1 sums u over the sequence; pass 2 forms
// the logits and accumulates F (rescaled by the running max), G, H for the tile; pass 3 applies
// X, Y to every query.
#include "device_common.hpp"
#include "launch.hpp"

namespace zeros {
namespace {

constexpr int kC = 32;
constexpr int kThreads = 256;
constexpr int kTile = 16;
constexpr int kTPR = 8;

template <int D>
struct EncSmem {
    float xh[kC][D + 1];   // normalised keys (pass 2) or queries (pass 3)
    float ub[kC][D + 1];   // u * ubar
    float vt[kC][kTile];
    float ubar[D];
    float F[D][kTile], G[D][kTile], Hs[D][kTile];
    float s[kC], w1[kC], wh[kC], w0[kC];
    float carry[4];
};

template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i) { return to_f32(p[i]); }

// Load rows [t0, t0+nval) of x into dst (normalised, optionally rotated); zero the rest.
template <int D, typename T, bool ROPE>
__device__ __forceinline__ void load_unit_rows(const T *x, int t0, int nval, float (*dst)[D + 1],
                                               const double *rope_rev) {
    constexpr int EPT = D / kTPR;
    const int tid = threadIdx.x;
    const int lr = tid / kTPR, c0 = (tid % kTPR) * EPT;
    const bool valid = lr < nval;
    const int tok = t0 + lr;
    float xv[EPT];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < EPT; ++c) {
        xv[c] = valid ? ld(x, static_cast<size_t>(tok) * D + c0 + c) : 0.f;
        ss += xv[c] * xv[c];
    }
    ss = group_sum<kTPR>(ss);
    const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int c = 0; c < EPT; ++c) xv[c] *= inv;
    if (ROPE) {
#pragma unroll
        for (int jj = 0; jj < EPT / 2; ++jj) {
            float cs, sn;
            rope_cos_sin(rope_rev[jj], tok, cs, sn);
            const float a = xv[2 * jj], b = xv[2 * jj + 1];
            xv[2 * jj] = a * cs - b * sn;
            xv[2 * jj + 1] = a * sn + b * cs;
        }
    }
#pragma unroll
    for (int c = 0; c < EPT; ++c) dst[lr][c0 + c] = xv[c];
}

template <int D, typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void encoder_valu_kernel(Problem p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    EncSmem<D> &sm = *reinterpret_cast<EncSmem<D> *>(smem_raw);
    constexpr int NTILE = D / kTile;
    constexpr int EPT = D / kTPR;
    const int tid = threadIdx.x;
    const int G = gridDim.x;
    int L = blockIdx.x;
    if ((G & 7) == 0) L = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int tile = L % NTILE;
    const int bh = L / NTILE;
    const int h = bh % p.H;
    const int N = p.N;
    const size_t row0 = static_cast<size_t>(bh) * N;
    const T *q = static_cast<const T *>(p.q) + row0 * D;
    const T *k = static_cast<const T *>(p.k) + row0 * D;
    const T *v = static_cast<const T *>(p.v) + row0 * D;
    const T *u = static_cast<const T *>(p.u) + row0 * D;
    const T *g1 = static_cast<const T *>(p.g1) + row0;
    const T *gh = static_cast<const T *>(p.gh) + row0;
    const T *g0 = p.g0 != nullptr ? static_cast<const T *>(p.g0) + row0 : nullptr;
    T *o = static_cast<T *>(p.o) + row0 * D;
    const float et = expf(p.tau[h]);
    const float rs_du = 1.f / sqrtf(static_cast<float>(D));
    const int lr = tid / kTPR, lp = tid % kTPR, c0 = lp * EPT;
    const float invN = 1.f / static_cast<float>(N);

    double rope_rev[ROPE ? EPT / 2 : 1];
    if (ROPE) {
#pragma unroll
        for (int jj = 0; jj < EPT / 2; ++jj) rope_rev[jj] = rope_rev_per_pos(c0 / 2 + jj, D, p.rope_base);
    }

    // ---- pass 1: ubar = (e^tau mu + sum u) / (e^tau + N)
    if (tid < D) {
        float su = 0.f;
        for (int n = 0; n < N; ++n) su += ld(u, static_cast<size_t>(n) * D + tid);
        sm.ubar[tid] = (et * p.mu[h * D + tid] + su) / (et + static_cast<float>(N));
    }
    for (int x = tid; x < D * kTile; x += kThreads) {
        (&sm.F[0][0])[x] = 0.f;
        (&sm.G[0][0])[x] = 0.f;
        (&sm.Hs[0][0])[x] = 0.f;
    }
    float m_c = kNegInf, E_c = 0.f, P_c = 0.f;
    __syncthreads();

    // ---- pass 2: logits, scalar sums and F, G, H for this tile
    for (int t0 = 0; t0 < N; t0 += kC) {
        const int nval = min(kC, N - t0);
        load_unit_rows<D, T, ROPE>(k, t0, nval, sm.xh, rope_rev);
        {
            const bool valid = lr < nval;
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                const float uv = valid ? ld(u, static_cast<size_t>(t0 + lr) * D + c0 + c) : 0.f;
                sm.ub[lr][c0 + c] = uv * sm.ubar[c0 + c];
            }
            const int r = tid / 8, mc = (tid % 8) * 2;
            const bool vv = r < nval;
            const size_t idx = static_cast<size_t>(t0 + r) * D + tile * kTile + mc;
            sm.vt[r][mc] = vv ? ld(v, idx) : 0.f;
            sm.vt[r][mc + 1] = vv ? ld(v, idx + 1) : 0.f;
        }
        __syncthreads();
        {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < EPT; ++c) acc += sm.ub[lr][c0 + c];
            acc = group_sum<kTPR>(acc);
            if (lp == 0) sm.s[lr] = -acc * rs_du;
        }
        __syncthreads();
        if (tid < 64) {
            const int r = tid;
            const bool valid = r < nval;
            const float sr = valid ? sm.s[r] : 0.f;
            float m = valid ? sr : kNegInf, e = valid ? 1.f : 0.f, ps = valid ? sr : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {   // full-wave reduction
                const float m2 = __shfl_xor(m, off, 64);
                const float e2 = __shfl_xor(e, off, 64);
                const float p2 = __shfl_xor(ps, off, 64);
                const float M = fmaxf(m, m2);
                e = e * exp_diff(m, M) + e2 * exp_diff(m2, M);
                ps += p2;
                m = M;
            }
            const float M = fmaxf(m_c, m);
            if (r == 0) {
                sm.carry[0] = M;
                sm.carry[1] = E_c * exp_diff(m_c, M) + e * exp_diff(m, M);
                sm.carry[2] = P_c + ps;
                sm.carry[3] = exp_diff(m_c, M);
            }
            if (r < kC) sm.w1[r] = valid ? expf(sr - M) : 0.f;
        }
        __syncthreads();
        {
            const int mm = tid % kTile;
            const float decay = sm.carry[3];
            for (int j = tid / kTile; j < D; j += kThreads / kTile) {
                float f = 0.f, g = 0.f, hh = 0.f;
                for (int i = 0; i < nval; ++i) {
                    const float kv = sm.xh[i][j] * sm.vt[i][mm];
                    f += sm.w1[i] * kv;
                    g += sm.s[i] * kv;
                    hh += kv;
                }
                sm.F[j][mm] = decay * sm.F[j][mm] + f;
                sm.G[j][mm] += g;
                sm.Hs[j][mm] += hh;
            }
        }
        m_c = sm.carry[0];
        E_c = sm.carry[1];
        P_c = sm.carry[2];
        __syncthreads();
    }

    // ---- X = F/E - H/N (in F), Y = G - (P/N) H (in G)
    {
        const float invE = 1.f / E_c;
        const float pn = P_c * invN;
        for (int x = tid; x < D * kTile; x += kThreads) {
            const float hh = (&sm.Hs[0][0])[x];
            (&sm.F[0][0])[x] = (&sm.F[0][0])[x] * invE - hh * invN;
            (&sm.G[0][0])[x] = (&sm.G[0][0])[x] - pn * hh;
        }
    }
    __syncthreads();

    // ---- pass 3: o_t = sigmah_t q^_t X + ((sigma1_t - sigmah_t)/N) q^_t Y (+ (sigma0_t/N) q^_t H)
    for (int t0 = 0; t0 < N; t0 += kC) {
        const int nval = min(kC, N - t0);
        load_unit_rows<D, T, ROPE>(q, t0, nval, sm.xh, rope_rev);
        if (tid < kC) {
            const bool valid = tid < nval;
            const float s1 = valid ? sigmoidf(ld(g1, t0 + tid)) : 0.f;
            const float sh = valid ? sigmoidf(ld(gh, t0 + tid)) : 0.f;
            sm.wh[tid] = sh;
            sm.w1[tid] = (s1 - sh) * invN;
            sm.w0[tid] = (valid && g0 != nullptr) ? sigmoidf(ld(g0, t0 + tid)) * invN : 0.f;
        }
        __syncthreads();
        {
            const int t = tid / 8, m0 = (tid % 8) * 2;
            float out[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int mm = m0 + x;
                float xX = 0.f, xY = 0.f, xH = 0.f;
                for (int j = 0; j < D; ++j) {
                    const float qv = sm.xh[t][j];
                    xX += qv * sm.F[j][mm];
                    xY += qv * sm.G[j][mm];
                    if (g0 != nullptr) xH += qv * sm.Hs[j][mm];
                }
                out[x] = sm.wh[t] * xX + sm.w1[t] * xY + sm.w0[t] * xH;
            }
            if (t < nval) {
                const size_t idx = static_cast<size_t>(t0 + t) * D + tile * kTile + m0;
                o[idx] = from_f32<T>(out[0]);
                o[idx + 1] = from_f32<T>(out[1]);
            }
        }
        __syncthreads();
    }
}

template <int D, typename T, bool ROPE>
hipError_t launch_one(const Problem &p, hipStream_t stream) {
    const size_t smem = sizeof(EncSmem<D>);
    const void *fn = reinterpret_cast<const void *>(&encoder_valu_kernel<D, T, ROPE>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(smem));
    if (err != hipSuccess) return err;
    const int grid = p.B * p.H * (D / kTile);
    hipLaunchKernelGGL((encoder_valu_kernel<D, T, ROPE>), dim3(grid), dim3(kThreads), smem, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem &p, hipStream_t stream) {
    if (p.dtype == ZEROS_BF16)
        return p.rope ? launch_one<D, bf16, true>(p, stream) : launch_one<D, bf16, false>(p, stream);
    return p.rope ? launch_one<D, float, true>(p, stream) : launch_one<D, float, false>(p, stream);
}

}  // namespace

// bfloat16 inputs with d 64 or 128 (d_u = d) run on the matrix cores; float32 inputs need the
// float32 arithmetic of this file (bfloat16 operands cannot meet their tolerance)
static bool encoder_uses_mfma(const Problem &p) {
    return p.dtype == ZEROS_BF16 && (p.d == 64 || p.d == 128) && p.du == p.d;
}

size_t encoder_work_bytes(const Problem &p) {
    return encoder_uses_mfma(p) && encoder_long_path(p) ? encoder_long_work_bytes(p) : 0;
}

hipError_t launch_encoder(const Problem &p, void *work, hipStream_t stream) {
    if (encoder_uses_mfma(p)) return encoder_long_path(p) ? launch_encoder_long(p, work, stream) : launch_encoder_mfma(p, stream);
    switch (p.d) {
        case 16: return launch_d<16>(p, stream);
        case 32: return launch_d<32>(p, stream);
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zeros
