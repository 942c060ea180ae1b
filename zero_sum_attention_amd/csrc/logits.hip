// Deviation logits of the causal ZeroS forward, computed ahead of the chunked scan.
//
// Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计 /
// 偏差 logits 设计: s_i = -(1/sqrt(d_u)) u_i . ubar_i with the prior-smoothed running mean
// ubar_i = (e^tau mu + sum_{j<=i} u_j) / (e^tau + i). The logit depends on the step i only, so
// all of them can be formed before the attention scan, in two passes over u:
//   pass 1 (useg_sum_kernel): per (head, segment of kSeg tokens), the column sums of u;
//   pass 2 (logits_stream_kernel for bfloat16 and d 64/128, logits_kernel otherwise): per
//                             (head, segment), the running sum starts from e^tau mu plus the
//                             sums of the earlier segments and gives ubar_i and s_i; for a
//                             sequence continued from a state, both also add the state's u-sum
//                             and token count.
// Output: s [B*H, N] float32, the per-segment sums [B*H, nseg, d_u] (their total is the u-sum of
// the recurrent state) and, per 64-token chunk, (max s, sum e^{s - max}, sum s) [B*H, nchunk, 4].
#include "device_common.hpp"
#include "launch.hpp"

namespace zeros {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&x)[8]);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16 *p, float (&x)[8]) {
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(a[i] << 16);
        x[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <typename T>
__device__ __forceinline__ void load4(const T *p, float (&x)[4]);
template <>
__device__ __forceinline__ void load4<bf16>(const bf16 *p, float (&x)[4]) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load4<float>(const float *p, float (&x)[4]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}

// Column sums of u over one segment: 8 consecutive features per thread, rows strided.
template <int D, typename T>
__global__ __launch_bounds__(kThreads) void useg_sum_kernel(const T *u, float *useg, int N, int nseg) {
    constexpr int VPR = D / 8;                 // threads per row
    constexpr int RPI = kThreads / VPR;        // rows per iteration
    __shared__ float part[RPI][D + 1];
    const int seg = blockIdx.x % nseg;
    const int bh = blockIdx.x / nseg;
    const int tid = threadIdx.x;
    const int c0 = (tid % VPR) * 8, rg = tid / VPR;
    const int r0 = seg * kLogitSeg, r1 = min(N, r0 + kLogitSeg);
    const T *ub = u + static_cast<size_t>(bh) * N * D;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // rows in flight per thread: the whole segment in one pass where the registers allow it. The
    // loads are unconditional (row index clamped, the extra rows not added): a load under a
    // per-row condition would wait for each row on its own.
    constexpr int U = kLogitSeg / RPI < (sizeof(T) == 2 ? 16 : 8) ? kLogitSeg / RPI : (sizeof(T) == 2 ? 16 : 8);
    for (int rb = r0 + rg; rb < r1; rb += U * RPI) {
        float x[U][8];
#pragma unroll
        for (int k = 0; k < U; ++k) load8(ub + static_cast<size_t>(min(rb + k * RPI, r1 - 1)) * D + c0, x[k]);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const bool ok = rb + k * RPI < r1;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += ok ? x[k][i] : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[rg][c0 + i] = acc[i];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
        for (int g = 0; g < RPI; ++g) s += part[g][tid];
        useg[(static_cast<size_t>(bh) * nseg + seg) * D + tid] = s;
    }
}

// Logits of one segment. Lane = token within a 64-token block, wave w = features
// [w*D/4, (w+1)*D/4). The running sum over the block is an inclusive lane scan per feature.
// su_in, t_in (both NULL, or both set): u sum and token count of earlier tokens of the sequence
// (a continued sequence), which join the prior.
template <int D, typename T>
__global__ __launch_bounds__(kThreads) void logits_kernel(const T *u, const float *mu, const float *tau,
                                                          const float *useg, float *s_out, float4 *agg,
                                                          int N, int H, int nseg, const float *su_in,
                                                          const int *t_in) {
    constexpr int DW = D / 4;                  // features per wave
    __shared__ float c0s[D];
    __shared__ float part[4][64];
    const int seg = blockIdx.x % nseg;
    const int bh = blockIdx.x / nseg;
    const int h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const float et = expf(tau[h]);
    const float tprev = t_in != nullptr ? static_cast<float>(t_in[bh]) : 0.f;
    if (tid < D) {
        const float s = et * mu[h * D + tid] + (su_in != nullptr ? su_in[static_cast<size_t>(bh) * D + tid] : 0.f);
        const float *us = useg + static_cast<size_t>(bh) * nseg * D + tid;
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // eight segment sums in flight
        for (int p0 = 0; p0 < seg; p0 += 8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] += p0 + j < seg ? us[static_cast<size_t>(p0 + j) * D] : 0.f;
        }
        c0s[tid] = s + (((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7])));
    }
    __syncthreads();
    float c0[DW], carry[DW];
#pragma unroll
    for (int i = 0; i < DW; ++i) {
        c0[i] = c0s[w * DW + i];
        carry[i] = 0.f;
    }
    const float rs_du = 1.f / sqrtf(static_cast<float>(D));
    const T *ub = u + static_cast<size_t>(bh) * N * D + w * DW;
    const int r0 = seg * kLogitSeg, r1 = min(N, r0 + kLogitSeg);
    // rows of the next 64-token block are read while this one is processed (clamped into the
    // sequence; rows past r1 are zeroed when used)
    float xn[DW];
    auto load_block = [&](const int b0) __attribute__((always_inline)) {
        const T *src = ub + static_cast<size_t>(min(b0 + lane, N - 1)) * D;
#pragma unroll
        for (int i = 0; i < DW; i += 4) {
            float y[4];
            load4(src + i, y);
#pragma unroll
            for (int a = 0; a < 4; ++a) xn[i + a] = y[a];
        }
    };
    if (r0 < r1) load_block(r0);
    for (int b0 = r0; b0 < r1; b0 += 64) {
        const int row = b0 + lane;
        const bool valid = row < r1;
        float x[DW], S[DW];
#pragma unroll
        for (int i = 0; i < DW; ++i) x[i] = valid ? xn[i] : 0.f;
        if (b0 + 64 < r1) load_block(b0 + 64);
#pragma unroll
        for (int i = 0; i < DW; ++i) S[i] = wave_scan_add(x[i]);
        const float inv = 1.f / (et + tprev + static_cast<float>(row + 1));
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < DW; ++i) {
            S[i] += carry[i];
            dot += x[i] * ((c0[i] + S[i]) * inv);
        }
        part[w][lane] = dot;
#pragma unroll
        for (int i = 0; i < DW; ++i) carry[i] = lane_f(S[i], 63);   // rows past r1 add zeros
        lds_barrier();
        if (w == 0) {
            const float tot = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
            const float sv = -tot * rs_du;
            if (valid) s_out[static_cast<size_t>(bh) * N + row] = sv;
            // aggregates of this 64-token chunk (segments are whole chunks)
            const float mx = lane_f(wave_scan_max(valid ? sv : kNegInf), 63);
            const float se = lane_f(wave_scan_add(valid ? __expf(sv - mx) : 0.f), 63);
            const float ss = lane_f(wave_scan_add(valid ? sv : 0.f), 63);
            if (lane == 0) agg[static_cast<size_t>(bh) * ((N + 63) / 64) + b0 / 64] = make_float4(mx, se, ss, 0.f);
        }
        lds_barrier();
    }
}

// Logits of one segment, bfloat16 u, by token streams: lane (stream st, feature group fg) keeps
// the running sum of features [8 fg, 8 fg + 8) over the TPS consecutive tokens of its stream (held
// in registers), so each token costs 3 float ops per feature. The stream starts are an exclusive
// scan of the stream sums: a shuffle scan over the streams of a wave (LPT lanes apart) plus the
// totals of the earlier waves and segments; the per-token dot partials of the LPT lanes of a
// stream are summed by a butterfly that leaves token k on lane k.
constexpr int kStreamThreads = 256;

template <int D>
__global__ __launch_bounds__(kStreamThreads, 4) void logits_stream_kernel(const bf16 *u, const float *mu, const float *tau,
                                                                 const float *useg, float *s_out, float4 *agg,
                                                                 int N, int H, int nseg, const float *su_in,
                                                                 const int *t_in) {
    constexpr int LPT = D / 8;                 // lanes per token row
    constexpr int NS = kStreamThreads / LPT;   // streams
    constexpr int TPS = kLogitSeg / NS;        // tokens per stream
    constexpr int NWV = kStreamThreads / 64;   // waves
    constexpr int G = kStreamThreads / D;      // threads per feature in the carry sum
    static_assert(TPS == LPT && kLogitSeg == kStreamThreads && D <= kStreamThreads, "stream shape");
    __shared__ float c0p[G][D];
    __shared__ float wtot[NWV][D];
    const int seg = blockIdx.x % nseg;
    const int bh = blockIdx.x / nseg;
    const int h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int st = tid / LPT, fg = tid % LPT, l = lane % LPT;
    // Loads in the order their values are needed, all before the first wait (loads complete in issue
    // order): the prior, the first kBatch G sums of the earlier segments, then this thread's token rows,
    // which stay in flight while the carry is summed. Every load is unconditional (index clamped,
    // the extra values not added): a load under a per-load condition waits on its own.
    const int f = tid % D, g = tid / D;        // carry sum: thread (feature f, phase g) adds segments g, g + G, ...
    const float *us = useg + static_cast<size_t>(bh) * nseg * D + f;
    const float et = expf(tau[h]);
    const float mu_f = mu[h * D + f];
    const float su_f = su_in != nullptr ? su_in[static_cast<size_t>(bh) * D + f] : 0.f;
    constexpr int kBatch = D == 128 ? 8 : 32;     // (registers: the token rows take 4 TPS)
    const int last = max(seg - 1, 0);
    float v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = us[static_cast<size_t>(min(g + j * G, last)) * D];
    const bf16 *ub = u + static_cast<size_t>(bh) * N * D;
    const int r0 = seg * kLogitSeg + st * TPS;
    uint4 x[TPS];
#pragma unroll
    for (int k = 0; k < TPS; ++k)
        x[k] = *reinterpret_cast<const uint4 *>(ub + static_cast<size_t>(min(r0 + k, N - 1)) * D + 8 * fg);
    {
        // prior (and the u-sum of a continued sequence's earlier tokens) plus the sums of u over the
        // earlier segments
        float a[8] = {g == 0 ? et * mu_f + su_f : 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kBatch; ++j) a[j % 8] += g + j * G < seg ? v[j] : 0.f;
        for (int q0 = g + kBatch * G; q0 < seg; q0 += 8 * G) {      // (more than kBatch G earlier segments)
            float v8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v8[j] = us[static_cast<size_t>(min(q0 + j * G, last)) * D];
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] += q0 + j * G < seg ? v8[j] : 0.f;
        }
        c0p[g][f] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    }
#pragma unroll
    for (int k = 0; k < TPS; ++k)
        if (r0 + k >= N) x[k] = make_uint4(0, 0, 0, 0);
    float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < TPS; ++k) {
        const uint32_t wv[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cs[2 * i] += __uint_as_float(wv[i] << 16);
            cs[2 * i + 1] += __uint_as_float(wv[i] & 0xffff0000u);
        }
    }
    // exclusive scan over the streams (in token order): the streams of a wave sit LPT lanes apart,
    // so a shuffle scan covers them; the totals of the earlier waves come through LDS
    float inc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float v = cs[i];
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) {
            const float t = __shfl_up(v, off, 64);
            if (lane >= off) v += t;
        }
        inc[i] = v;
    }
    if (lane >= 64 - LPT) {
#pragma unroll
        for (int i = 0; i < 8; ++i) wtot[wave][8 * fg + i] = inc[i];
    }
    __syncthreads();
    float R[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int f = 8 * fg + i;
        float c = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) c += c0p[g][f];
#pragma unroll
        for (int w2 = 0; w2 < NWV; ++w2) c += w2 < wave ? wtot[w2][f] : 0.f;
        const float ex = __shfl_up(inc[i], LPT, 64);      // streams of this wave before this one
        R[i] = lane >= LPT ? c + ex : c;
    }
    // the packed rows go through an empty asm: the dot pass unpacks them again instead of the
    // compiler holding both the packed and the unpacked values (twice the registers) since the sums
#pragma unroll
    for (int k = 0; k < TPS; ++k) asm volatile("" : "+v"(x[k].x), "+v"(x[k].y), "+v"(x[k].z), "+v"(x[k].w));
    float d[TPS];                              // per-token dot partials, reduced in place below
#pragma unroll
    for (int k = 0; k < TPS; ++k) {
        const uint32_t wv[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = __uint_as_float(wv[i] << 16), b = __uint_as_float(wv[i] & 0xffff0000u);
            R[2 * i] += a;
            R[2 * i + 1] += b;
            acc = fmaf(a, R[2 * i], acc);
            acc = fmaf(b, R[2 * i + 1], acc);
        }
        d[k] = acc;
    }
    // butterfly over the LPT lanes of a stream: token l of the stream ends on lane l. A stream is LPT
    // tokens, so wave w then holds tokens 64 w + lane of the segment: one 64-token chunk, whose
    // logits and aggregate (max, sum e^{s - max}, sum s) are written straight from the registers.
#pragma unroll
    for (int off = LPT / 2; off >= 1; off >>= 1) {
        const bool hi = (l & off) != 0;
#pragma unroll
        for (int i = 0; i < off; ++i) {
            const float keep = hi ? d[off + i] : d[i];
            const float send = hi ? d[i] : d[off + i];
            d[i] = keep + __shfl_xor(send, off, 64);
        }
    }
    const int c0 = seg * kLogitSeg + 64 * wave;          // first token of this wave's chunk
    if (c0 < N) {
        const int row = c0 + lane;
        const bool valid = row < N;
        // (tokens of a continued sequence are positions t_in + 1 ...; read here, where it is used)
        const float tprev = t_in != nullptr ? static_cast<float>(t_in[bh]) : 0.f;
        const float s = -d[0] * (1.f / sqrtf(static_cast<float>(D))) / (et + tprev + static_cast<float>(row + 1));
        if (valid) s_out[static_cast<size_t>(bh) * N + row] = s;
        const float mx = lane_f(wave_scan_max(valid ? s : kNegInf), 63);
        const float se = lane_f(wave_scan_add(valid ? __expf(s - mx) : 0.f), 63);
        const float ss = lane_f(wave_scan_add(valid ? s : 0.f), 63);
        if (lane == 0) agg[static_cast<size_t>(bh) * ((N + 63) / 64) + c0 / 64] = make_float4(mx, se, ss, 0.f);
    }
}

// Logits of a short sequence (N <= lh_max_n<D>()) in one pass over u: one workgroup of 1024 threads
// per head. Thread (feature group fg of 4 features, token block tb of TB tokens) reads its TB rows
// once; the block totals go through LDS for an exclusive prefix over the blocks (each thread adds 4
// block totals, then the parts before it), which gives every thread the running sum at its first
// token; the per-token dots are summed over the FG lanes of a row by DPP. The 256-token segment sums
// and the 64-token (max, sum e^{s - max}, sum s) aggregates come from the same data. The token
// blocks are fixed (TB per d), so the grouping, and the rounding, do not depend on N.
constexpr int kLHThreads = 1024;
template <int D> __host__ __device__ constexpr int lh_tb() { return D == 16 ? 4 : D == 32 ? 8 : 16; }
template <int D> __host__ __device__ constexpr int lh_max_n() { return kLHThreads / (D / 4) * lh_tb<D>(); }

template <int D, typename T>
__global__ __launch_bounds__(kLHThreads) void logits_head_kernel(const T *u, const float *mu, const float *tau,
                                                                 float *useg, float *s_out, float4 *agg, int N,
                                                                 int H, int nseg, const float *su_in,
                                                                 const int *t_in) {
    constexpr int FG = D / 4;              // feature groups = threads per token row
    constexpr int TBN = kLHThreads / FG;   // token blocks
    constexpr int TB = lh_tb<D>();         // tokens per block
    constexpr int P = kLHThreads / D;      // parts of the block prefix per feature (4 blocks each)
    static_assert(TBN == 4 * P && 64 % TB == 0 && kLogitSeg % TB == 0, "per-head logits shape");
    __shared__ float colp[TBN][D];         // block totals, then their exclusive prefix
    __shared__ float psum[P][D];           // totals of 4 blocks
    __shared__ float4 aggp[TBN];           // (max, sum e^{s - max}, sum s) of each block
    // (the barriers order LDS only: a full barrier would also wait for the logit and u-sum stores)
    const int bh = blockIdx.x, h = bh % H;
    const int tid = threadIdx.x, fg = tid % FG, tb = tid / FG;
    const T *ub = u + static_cast<size_t>(bh) * N * D;
    const int t0 = tb * TB;
    float x[TB][4];
#pragma unroll
    for (int k = 0; k < TB; ++k) {
        const int t = t0 + k;
        float y[4];
        load4(ub + static_cast<size_t>(min(t, N - 1)) * D + 4 * fg, y);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[k][i] = t < N ? y[i] : 0.f;
    }
    float tot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < TB; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] += x[k][i];
    *reinterpret_cast<float4 *>(&colp[tb][4 * fg]) = make_float4(tot[0], tot[1], tot[2], tot[3]);
    lds_barrier();
    {
        // thread (f, part): blocks 4 part .. 4 part + 3 of feature f
        const int f = tid % D, part = tid / D;
        float a[4], run = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = colp[4 * part + e][f];
            run += a[e];
        }
        psum[part][f] = run;
        lds_barrier();
        float pre = 0.f;
        for (int q = 0; q < part; ++q) pre += psum[q][f];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            colp[4 * part + e][f] = pre;      // exclusive prefix of block 4 part + e
            pre += a[e];
        }
        // u sums of the 256-token segments: the prefix difference at their block boundaries
        lds_barrier();
        if (part < nseg) {
            constexpr int BPS = kLogitSeg / TB;            // blocks per segment
            const int b0 = part * BPS, b1 = b0 + BPS;
            float hi = 0.f;
            if (b1 < TBN) hi = colp[b1][f];
            else                                            // the prefix past the last block: all of it
                for (int q = 0; q < P; ++q) hi += psum[q][f];
            useg[(static_cast<size_t>(bh) * nseg + part) * D + f] = hi - colp[b0][f];
        }
    }
    // logits of this thread's tokens
    const float et = expf(tau[h]);
    const float tprev = t_in != nullptr ? static_cast<float>(t_in[bh]) : 0.f;
    float run[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int f = 4 * fg + i;
        run[i] = et * mu[h * D + f] + (su_in != nullptr ? su_in[static_cast<size_t>(bh) * D + f] : 0.f) + colp[tb][f];
    }
    const float rs_du = 1.f / sqrtf(static_cast<float>(D));
    float m = kNegInf, ps = 0.f;
    float sv[TB];
#pragma unroll
    for (int k = 0; k < TB; ++k) {
        const int t = t0 + k;
        const float inv = 1.f / (et + tprev + static_cast<float>(t + 1));
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            run[i] += x[k][i];
            dot += x[k][i] * (run[i] * inv);
        }
        dot = group_sum<FG>(dot);
        sv[k] = -dot * rs_du;
        if (t < N) {
            if (fg == 0) s_out[static_cast<size_t>(bh) * N + t] = sv[k];
            m = fmaxf(m, sv[k]);
            ps += sv[k];
        }
    }
    float e = 0.f;
#pragma unroll
    for (int k = 0; k < TB; ++k)
        if (t0 + k < N) e += __expf(sv[k] - m);
    if (fg == 0) aggp[tb] = make_float4(m, e, ps, 0.f);
    lds_barrier();
    // 64-token aggregates: 64 / TB blocks each
    const int nb64 = (N + 63) / 64;
    if (tid < nb64) {
        float M = kNegInf, E = 0.f, Ps = 0.f;
#pragma unroll
        for (int j = 0; j < 64 / TB; ++j) {
            const float4 a = aggp[tid * (64 / TB) + j];
            const float mx = fmaxf(M, a.x);
            E = (M == kNegInf ? 0.f : E * __expf(M - mx)) + (a.x == kNegInf ? 0.f : a.y * __expf(a.x - mx));
            M = mx;
            Ps += a.z;
        }
        agg[static_cast<size_t>(bh) * nb64 + tid] = make_float4(M, E, Ps, 0.f);
    }
}

template <int D, typename T>
hipError_t launch_t(const Problem &p, float *useg, float *s_out, float4 *agg, hipStream_t stream) {
    const int nseg = (p.N + kLogitSeg - 1) / kLogitSeg;
    // short sequences in one pass per head (the float32 path; the bfloat16 matrix-core path keeps
    // its stream kernel)
    if constexpr (sizeof(T) == 4) {
        if (p.N <= lh_max_n<D>()) {
            hipLaunchKernelGGL((logits_head_kernel<D, T>), dim3(p.B * p.H), dim3(kLHThreads), 0, stream,
                               static_cast<const T *>(p.u), p.mu, p.tau, useg, s_out, agg, p.N, p.H, nseg,
                               p.sin.Su, p.sin.t);
            return hipGetLastError();
        }
    }
    const int grid = p.B * p.H * nseg;
    hipLaunchKernelGGL((useg_sum_kernel<D, T>), dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const T *>(p.u), useg, p.N, nseg);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // (a continued sequence passes the state's u-sum and token count, which join the prior)
    if constexpr (sizeof(T) == 2 && (D == 64 || D == 128)) {
        hipLaunchKernelGGL((logits_stream_kernel<D>), dim3(grid), dim3(kStreamThreads), 0, stream,
                           static_cast<const bf16 *>(p.u), p.mu, p.tau, useg, s_out, agg, p.N, p.H, nseg,
                           p.sin.Su, p.sin.t);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((logits_kernel<D, T>), dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const T *>(p.u), p.mu, p.tau, useg, s_out, agg, p.N, p.H, nseg,
                       p.sin.Su, p.sin.t);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem &p, float *useg, float *s_out, float4 *agg, hipStream_t stream) {
    return p.dtype == ZEROS_BF16 ? launch_t<D, bf16>(p, useg, s_out, agg, stream)
                                 : launch_t<D, float>(p, useg, s_out, agg, stream);
}

}  // namespace

hipError_t launch_usum(const Problem &p, float *useg, hipStream_t stream) {
    if (p.N == 0) return hipSuccess;
    const int nseg = (p.N + kLogitSeg - 1) / kLogitSeg;
    const dim3 grid(p.B * p.H * nseg);
    const bool bf = p.dtype == ZEROS_BF16;
    switch (p.d) {
        case 64:
            if (bf) hipLaunchKernelGGL((useg_sum_kernel<64, bf16>), grid, dim3(kThreads), 0, stream, static_cast<const bf16 *>(p.u), useg, p.N, nseg);
            else hipLaunchKernelGGL((useg_sum_kernel<64, float>), grid, dim3(kThreads), 0, stream, static_cast<const float *>(p.u), useg, p.N, nseg);
            break;
        case 128:
            if (bf) hipLaunchKernelGGL((useg_sum_kernel<128, bf16>), grid, dim3(kThreads), 0, stream, static_cast<const bf16 *>(p.u), useg, p.N, nseg);
            else hipLaunchKernelGGL((useg_sum_kernel<128, float>), grid, dim3(kThreads), 0, stream, static_cast<const float *>(p.u), useg, p.N, nseg);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_logits(const Problem &p, float *useg, float *s_out, float4 *agg, hipStream_t stream) {
    if (p.N == 0) return hipSuccess;
    switch (p.d) {
        case 16: return launch_d<16>(p, useg, s_out, agg, stream);
        case 32: return launch_d<32>(p, useg, s_out, agg, stream);
        case 64: return launch_d<64>(p, useg, s_out, agg, stream);
        case 128: return launch_d<128>(p, useg, s_out, agg, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zeros
