// One recurrent ZeroS step per (sequence, head), state updated in place.
//
// Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计 /
// 线性时间前缀扫描: each new token costs O(d^2) on the d x d prefix states. For the token at
// position t (1-based):
//   S_u += u;  ubar = (e^tau mu + S_u)/(e^tau + t);  s = -(u . ubar)/sqrt(d_u)
//   m' = max(m, s); c = e^{m - m'}; E' = c E + e^{s - m'}; P' = P + s
//   F' = c F + e^{s - m'} k^^T v;  G' = G + s k^^T v;  H' = H + k^^T v
//   o = q^ (sigmah/E' F' + ((sigma1 - sigmah)/t) G' + (-(sigma1 - sigmah) P'/t^2 - sigmah/t) H')
// The step is a pure stream over the 3 d^2 floats of state: one workgroup per (sequence, head)
// reads and writes them with 16-byte accesses along the value index.
#include "device_common.hpp"
#include "launch.hpp"

namespace zeros {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i) { return to_f32(p[i]); }

template <int D, typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void decode_kernel(Problem p) {
    constexpr int C4 = D / 4;                 // float4 units per state row
    constexpr int UNITS = D * C4;             // float4 units per state matrix
    __shared__ float qh[D], kh[D], vv[D], red[kThreads];
    __shared__ float partial[kThreads][4];
    __shared__ float coef[6];                 // c, e, s, a, beta, gamma

    const int tid = threadIdx.x;
    const int sh_idx = blockIdx.x;            // sequence * H + head
    const int h = sh_idx % p.H;
    const T *q = static_cast<const T *>(p.q) + static_cast<size_t>(sh_idx) * D;
    const T *k = static_cast<const T *>(p.k) + static_cast<size_t>(sh_idx) * D;
    const T *v = static_cast<const T *>(p.v) + static_cast<size_t>(sh_idx) * D;
    const T *u = static_cast<const T *>(p.u) + static_cast<size_t>(sh_idx) * D;
    T *o = static_cast<T *>(p.o) + static_cast<size_t>(sh_idx) * D;
    const int t_old = p.st.t[sh_idx];
    const float tn = static_cast<float>(t_old + 1);
    const float et = expf(p.tau[h]);

    // ---- token vectors: q^, k^ (wave 0 and wave 1), v; u . ubar partials
    float prod = 0.f;
    if (tid < D) {
        const float uj = ld(u, tid);
        float *Su = p.st.Su + static_cast<size_t>(sh_idx) * D;
        const float su = Su[tid] + uj;
        Su[tid] = su;
        prod = uj * ((et * p.mu[h * D + tid] + su) / (et + tn));
        vv[tid] = ld(v, tid);
    }
    red[tid] = prod;
    {
        // normalise q (threads 0..63) and k (threads 64..127); each lane covers D/64 entries
        constexpr int PER = (D + 63) / 64;
        const int lane = tid & 63;
        const int which = tid >> 6;
        if (which < 2) {
            const T *src = which == 0 ? q : k;
            float x[PER];
            float ss = 0.f;
#pragma unroll
            for (int a = 0; a < PER; ++a) {
                const int j = lane * PER + a;
                x[a] = j < D ? ld(src, j) : 0.f;
                ss += x[a] * x[a];
            }
            ss = group_sum<64>(ss);
            const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
            float *dst = which == 0 ? qh : kh;
#pragma unroll
            for (int a = 0; a < PER; ++a) {
                const int j = lane * PER + a;
                if (j < D) dst[j] = x[a] * inv;
            }
        }
    }
    __syncthreads();
    if (ROPE) {
        // pair jp of q (even threads) or k (odd threads), rotated by position t_old (0-based)
        const int jp = tid >> 1;
        const bool mine = tid < D;
        float *x = (tid & 1) ? kh : qh;
        float cs = 1.f, sn = 0.f, a = 0.f, b = 0.f;
        if (mine) {
            rope_cos_sin(rope_rev_per_pos(jp, D, p.rope_base), t_old, cs, sn);
            a = x[2 * jp];
            b = x[2 * jp + 1];
        }
        __syncthreads();
        if (mine) {
            x[2 * jp] = a * cs - b * sn;
            x[2 * jp + 1] = a * sn + b * cs;
        }
        __syncthreads();
    }
    if (tid < 64) {
        float acc = 0.f;
        for (int j = tid; j < kThreads; j += 64) acc += red[j];
        acc = group_sum<64>(acc);
        if (tid == 0) {
            const float s = -acc / sqrtf(static_cast<float>(D));
            const float m_old = p.st.m[sh_idx];
            const float m_new = fmaxf(m_old, s);
            const float c = exp_diff(m_old, m_new);
            const float e = expf(s - m_new);
            const float E = c * p.st.E[sh_idx] + e;
            const float P = p.st.P[sh_idx] + s;
            const float s1 = sigmoidf(ld(static_cast<const T *>(p.g1), sh_idx));
            const float sgh = sigmoidf(ld(static_cast<const T *>(p.gh), sh_idx));
            const float d1 = s1 - sgh;
            coef[0] = c;
            coef[1] = e;
            coef[2] = s;
            coef[3] = sgh / E;
            coef[4] = d1 / tn;
            // the optional zero-order gate adds sigma0_t / t to gamma
            const float s0 = p.g0 != nullptr ? sigmoidf(ld(static_cast<const T *>(p.g0), sh_idx)) : 0.f;
            coef[5] = -d1 * (P / tn) / tn + (s0 - sgh) / tn;
            p.st.m[sh_idx] = m_new;
            p.st.E[sh_idx] = E;
            p.st.P[sh_idx] = P;
            p.st.t[sh_idx] = t_old + 1;
        }
    }
    __syncthreads();

    // ---- stream the three states
    const float c = coef[0], e = coef[1], s = coef[2], a = coef[3], b = coef[4], g = coef[5];
    const size_t mat0 = static_cast<size_t>(sh_idx) * D * D;
    float4 *F = reinterpret_cast<float4 *>(p.st.F + mat0);
    float4 *G = reinterpret_cast<float4 *>(p.st.G + mat0);
    float4 *Hm = reinterpret_cast<float4 *>(p.st.Hs + mat0);
    const int c4 = tid % C4;
    const float4 v4 = make_float4(vv[4 * c4], vv[4 * c4 + 1], vv[4 * c4 + 2], vv[4 * c4 + 3]);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int x = tid; x < UNITS; x += kThreads) {
        const int j = x / C4;
        const float kj = kh[j], qj = qh[j];
        float4 f = F[x], gg = G[x], hh = Hm[x];
        const float kv[4] = {kj * v4.x, kj * v4.y, kj * v4.z, kj * v4.w};
        float *fp = &f.x, *gp = &gg.x, *hp = &hh.x;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            fp[y] = c * fp[y] + e * kv[y];
            gp[y] = gp[y] + s * kv[y];
            hp[y] = hp[y] + kv[y];
            acc[y] += qj * (a * fp[y] + b * gp[y] + g * hp[y]);
        }
        F[x] = f;
        G[x] = gg;
        Hm[x] = hh;
    }
#pragma unroll
    for (int y = 0; y < 4; ++y) partial[tid][y] = acc[y];
    __syncthreads();
    if (tid < D) {
        const int cc = tid / 4, y = tid % 4;
        float sum = 0.f;
        for (int r = cc; r < kThreads; r += C4) sum += partial[r][y];
        o[tid] = from_f32<T>(sum);
    }
}

template <int D, typename T, bool ROPE>
hipError_t launch_one(const Problem &p, hipStream_t stream) {
    hipLaunchKernelGGL((decode_kernel<D, T, ROPE>), dim3(p.B * p.H), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem &p, hipStream_t stream) {
    if (p.dtype == ZEROS_BF16)
        return p.rope ? launch_one<D, bf16, true>(p, stream) : launch_one<D, bf16, false>(p, stream);
    return p.rope ? launch_one<D, float, true>(p, stream) : launch_one<D, float, false>(p, stream);
}

}  // namespace

hipError_t launch_decode(const Problem &p, hipStream_t stream) {
    switch (p.d) {
        case 16: return launch_d<16>(p, stream);
        case 32: return launch_d<32>(p, stream);
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zeros
