// Encoder (non-causal) ZeroS forward for long bfloat16 sequences (encoder_long_path, d in
// {64, 128}), token-parallel.
//
// Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", 关键设计 with
// t = N for every query (the encoder form): o_t = sigmah_t q^_t X + ((sigma1_t - sigmah_t)/N) q^_t Y
// (+ (sigma0_t/N) q^_t H with the zero-order gate), X = sum_i (e^{s_i - m}/E - 1/N) k^_i^T v_i,
// Y = sum_i (s_i - P/N) k^_i^T v_i, H = sum_i k^_i^T v_i, and the logits of 偏差 logits 设计 over
// the global prior-smoothed mean ubar. Every quantity is a sum over the tokens, so the sequence is
// cut into blocks and each launch runs one workgroup per (batch, head, block):
//   1. column sums of u per 256-token block (logits.hip);
//   2. ubar from those sums; per state block of SB tokens its logits and (max, sum e^{s - max}, sum s);
//   3. per state block the merged (m, E, P) of the head, unit k^ and v w_X, v w_Y (v) staged in LDS,
//      and the block's partial X, Y (H) on the matrix cores, written as float32;
//   4. X, Y (H) = the sum of the partials in block order, stored as bf16 X^T, Y^T (H^T);
//   5. per output block the outputs from q^ and X^T, Y^T (H^T) on the matrix cores.
// A state block holds SB = 256 spb tokens, spb a power of two up to 8 chosen so that the grid still
// has about 512 workgroups: the partials cost 3 d^2 floats per block, against 4 SB d bytes of k, v.
// Scratch: encoder_long_work_bytes(p).
#include "device_common.hpp"
#include "encoder_common.hpp"
#include "kv_states.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace zeros {
namespace {

constexpr int kLB = kLogitSeg;     // tokens per u-sum block
constexpr int kLPad = 8;           // bf16 elements of row padding in LDS (rows stay 4 mod 8 words)
constexpr int kLThreads = 256;     // logits kernel

template <int D> constexpr int out_threads() { return D == 64 ? 256 : 512; }
template <int D> constexpr int out_block() { return D == 64 ? 512 : 1024; }

struct LongPlan {
    int nblk;   // 256-token u-sum blocks
    int spb;    // u-sum blocks per state block
    int nsb;    // state blocks
};

LongPlan long_plan(const Problem &p) {
    LongPlan lp{};
    const long bh = static_cast<long>(p.B) * p.H;
    lp.nblk = (p.N + kLB - 1) / kLB;
    lp.spb = 1;
    while (lp.spb < 8 && bh * ((lp.nblk + 2 * lp.spb - 1) / (2 * lp.spb)) >= 512) lp.spb *= 2;
    lp.nsb = (lp.nblk + lp.spb - 1) / lp.spb;
    return lp;
}

struct LongWork {
    float *usum;       // [B H, nblk, d] u sums per 256-token block
    float *s;          // [B H, N] logits
    float4 *aggb;      // [B H, nsb] (max, sum e^{s - max}, sum s) per state block
    float *xpart;      // [B H, nsb, 3, d (column c), d (feature f)] partial X, Y, H, transposed
    uint16_t *xt;      // [B H, 3, d (c), d (f)] X^T, Y^T, H^T as bf16
    int nblk, nsb, sb_tokens;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

struct Sizes {
    size_t usum, s, aggb, xpart, xt;
};
Sizes sizes(const Problem &p, const LongPlan &lp) {
    const size_t bh = static_cast<size_t>(p.B) * p.H, d = p.d;
    return {up256(bh * lp.nblk * d * 4), up256(bh * p.N * 4), up256(bh * lp.nsb * 16),
            up256(bh * lp.nsb * 3 * d * d * 4), up256(bh * 3 * d * d * 2)};
}

LongWork carve(void *base, const Problem &p) {
    const LongPlan lp = long_plan(p);
    const Sizes z = sizes(p, lp);
    char *b = static_cast<char *>(base);
    LongWork w{};
    w.usum = reinterpret_cast<float *>(b);
    w.s = reinterpret_cast<float *>(b += z.usum);
    w.aggb = reinterpret_cast<float4 *>(b += z.s);
    w.xpart = reinterpret_cast<float *>(b += z.aggb);
    w.xt = reinterpret_cast<uint16_t *>(b += z.xpart);
    w.nblk = lp.nblk;
    w.nsb = lp.nsb;
    w.sb_tokens = lp.spb * kLB;
    return w;
}

// ---- 2: ubar, the logits of a state block and its (max, sum e^{s - max}, sum s). Passes of CT
// tokens, 8 rows per thread, the next pass's rows loaded before the current one is used.
template <int D>
__global__ __launch_bounds__(kLThreads) void enc_long_logits_kernel(Problem p, LongWork w) {
    constexpr int LPR = D / 8, RPP = kLThreads / LPR, NP = 8, CT = RPP * NP;
    __shared__ float ubar[D];
    __shared__ float4 red[kLThreads / 64];
    const int nsb = w.nsb, sb = blockIdx.x % nsb, bh = blockIdx.x / nsb, h = bh % p.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fr = tid % LPR, rr = tid / LPR;
    const int N = p.N, t0 = sb * w.sb_tokens, t1 = min(N, t0 + w.sb_tokens);
    const uint16_t *u = static_cast<const uint16_t *>(p.u) + static_cast<size_t>(bh) * N * D;
    uint4 ur[NP];
    auto load = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NP; ++j)
            ur[j] = *reinterpret_cast<const uint4 *>(u + static_cast<size_t>(min(c0 + rr + RPP * j, N - 1)) * D + 8 * fr);
    };
    load(t0);
    if (tid < D) {
        // the head's block sums: unconditional loads (index clamped, the extra ones weighted 0)
        const int nblk = w.nblk;
        const float *us = w.usum + static_cast<size_t>(bh) * nblk * D + tid;
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < nblk; j0 += 8) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                a[jj] += (j0 + jj < nblk ? 1.f : 0.f) * us[static_cast<size_t>(min(j0 + jj, nblk - 1)) * D];
        }
        const float su = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
        const float et = expf(p.tau[h]);
        ubar[tid] = (et * p.mu[h * D + tid] + su) / (et + static_cast<float>(N));
    }
    __syncthreads();
    float ub[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ub[i] = ubar[8 * fr + i];
    const float rs_du = 1.f / sqrtf(static_cast<float>(D));
    float m = kNegInf, e = 0.f, ps = 0.f;
    float *srow = w.s + static_cast<size_t>(bh) * N;
    for (int c0 = t0; c0 < t1; c0 += CT) {
        float x[NP][8];
#pragma unroll
        for (int j = 0; j < NP; ++j) unpack8(ur[j], x[j]);
        if (c0 + CT < t1) load(c0 + CT);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int r = c0 + rr + RPP * j;
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) dot = fmaf(x[j][i], ub[i], dot);
            dot = group_sum<LPR>(dot);
            if (r < t1 && fr == 0) {
                const float sv = -dot * rs_du;
                srow[r] = sv;
                lse_merge(m, e, sv, 1.f);
                ps += sv;
            }
        }
    }
    wave_lse_merge(m, e, ps);
    if (lane == 0) red[wv] = make_float4(m, e, ps, 0.f);
    __syncthreads();
    if (tid == 0) {
        float M = kNegInf, E = 0.f, P = 0.f;
#pragma unroll
        for (int i = 0; i < kLThreads / 64; ++i) {
            lse_merge(M, E, red[i].x, red[i].y);
            P += red[i].z;
        }
        w.aggb[static_cast<size_t>(bh) * nsb + sb] = make_float4(M, E, P, 0.f);
    }
}

// ---- 3: the partial states of a state block (kv_states.hpp), with the weights of the whole head:
// w_X = e^{s - m}/E - 1/N, w_Y = s - P/N, from the merged state-block aggregates.
template <int D, bool ROPE, int NS>
__global__ __launch_bounds__(kv_threads<D>()) void enc_long_state_kernel(Problem p, LongWork w) {
    __shared__ __align__(16) KvSmem<D, NS> sm;
    __shared__ float scal[3];
    __shared__ double rev[ROPE ? D / 2 : 1];
    const int nsb = w.nsb, sb = blockIdx.x % nsb, bh = blockIdx.x / nsb;
    const int N = p.N, t0 = sb * w.sb_tokens, t1 = min(N, t0 + w.sb_tokens);
    const size_t row0 = static_cast<size_t>(bh) * N;
    KvStates<D, ROPE, NS> kv(sm, static_cast<const uint16_t *>(p.k) + row0 * D, static_cast<const uint16_t *>(p.v) + row0 * D,
                             w.s + row0, rev, N, t0, t1, 0);
    kv.start();
    if (ROPE && kv.tid < D / 2) rev[kv.tid] = rope_rev_per_pos(kv.tid, D, p.rope_base);
    if (kv.wv == 0) {                  // (m, E, P) of the head from the state-block aggregates
        float m = kNegInf, e = 0.f, ps = 0.f;
        for (int j = kv.lane; j < nsb; j += 64) {
            const float4 a = w.aggb[static_cast<size_t>(bh) * nsb + j];
            lse_merge(m, e, a.x, a.y);
            ps += a.z;
        }
        wave_lse_merge(m, e, ps);
        if (kv.lane == 0) {
            scal[0] = m;
            scal[1] = e;
            scal[2] = ps;
        }
    }
    lds_barrier();
    const float M = scal[0], invE = scal[1] > 0.f ? 1.f / scal[1] : 0.f;
    const float invN = 1.f / static_cast<float>(N), PN = scal[2] * invN;
    kv.run([&](float sv) __attribute__((always_inline)) { return make_float2(__expf(sv - M) * invE - invN, sv - PN); });
    // accumulator lane (l16, g4) of tile ft holds features 16 ft + 4 g4 + [0, 4) of column 16 wv + l16
    float *xp = w.xpart + (static_cast<size_t>(bh) * nsb + sb) * 3 * D * D;
#pragma unroll
    for (int ft = 0; ft < D / 16; ++ft) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
            *reinterpret_cast<float4 *>(xp + static_cast<size_t>(s) * D * D + static_cast<size_t>(16 * kv.wv + kv.l16) * D + 16 * ft +
                                        4 * kv.g4) = make_float4(kv.acc[s][ft][0], kv.acc[s][ft][1], kv.acc[s][ft][2], kv.acc[s][ft][3]);
    }
}

// ---- 4: the states as the sum of the state-block partials (in block order), stored as bf16
// X^T, Y^T (H^T); 4 consecutive elements per thread
__global__ __launch_bounds__(256) void enc_long_reduce_kernel(LongWork w, int dd, int ns) {
    const int bh = blockIdx.x, e = 4 * (blockIdx.y * 256 + threadIdx.x);
    if (e >= ns * dd) return;
    const int nsb = w.nsb;
    const float *xp = w.xpart + static_cast<size_t>(bh) * nsb * 3 * dd + e;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < nsb; ++j) {
        const float4 x = *reinterpret_cast<const float4 *>(xp + static_cast<size_t>(j) * 3 * dd);
        a.x += x.x;
        a.y += x.y;
        a.z += x.z;
        a.w += x.w;
    }
    *reinterpret_cast<uint2 *>(w.xt + static_cast<size_t>(bh) * 3 * dd + e) = make_uint2(pack2(a.x, a.y), pack2(a.z, a.w));
}

// ---- 5: the outputs of an output block of OB tokens; wave w takes its 16-token steps w, w + NW, ...
// with the queries of the next two steps in flight
template <int D, bool ROPE, int NS>
__global__ __launch_bounds__(out_threads<D>()) void enc_long_out_kernel(Problem p, LongWork w) {
    constexpr int NT = out_threads<D>(), NW = NT / 64, OB = out_block<D>(), SPW = OB / 16 / NW;
    constexpr int KS = D / 32, NFT = D / 16;
    __shared__ __align__(16) uint16_t sxy[NS][D][D + kLPad];
    __shared__ double rev[ROPE ? D / 2 : 1];
    const int N = p.N, nob = (N + OB - 1) / OB;
    const int ob = blockIdx.x % nob, bh = blockIdx.x / nob;
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int t0 = ob * OB;
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint16_t *q = static_cast<const uint16_t *>(p.q) + row0 * D;
    const uint16_t *g1 = static_cast<const uint16_t *>(p.g1) + row0;
    const uint16_t *gh = static_cast<const uint16_t *>(p.gh) + row0;
    const uint16_t *g0 = NS == 3 ? static_cast<const uint16_t *>(p.g0) + row0 : nullptr;
    uint16_t *o = static_cast<uint16_t *>(p.o) + row0 * D;
    // the queries and gates of one step in registers; loads of steps past the block re-read its last
    // step (from L2) so that every load is unconditional
    struct Qs {
        uint4 q[KS];
        uint32_t g1, gh, g0;
    };
    auto load = [&](Qs &x, int st) __attribute__((always_inline)) {
        st = min(st, SPW - 1);
        const int tq = min(t0 + 16 * (wv + NW * st) + l16, N - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) x.q[ks] = *reinterpret_cast<const uint4 *>(q + static_cast<size_t>(tq) * D + 32 * ks + 8 * g4);
        x.g1 = g1[tq];
        x.gh = gh[tq];
        x.g0 = NS == 3 ? g0[tq] : 0u;
    };
    Qs qs0, qs1;
    load(qs0, 0);
    load(qs1, 1);
    // X^T, Y^T (H^T) into LDS, 16 bytes per thread and step. Row 16 ct + 4 g + i of the LDS copy holds
    // column c = (D/4) g + 4 ct + i, so that the output tiles ct = 0 .. D/16 - 1 give lane (l16, g4)
    // the D/4 consecutive columns (D/4) g4 + [0, D/4) of its token, stored as whole 16-byte pieces.
    const uint16_t *xt = w.xt + static_cast<size_t>(bh) * 3 * D * D;
    for (int x = tid; x < NS * D * D / 8; x += NT) {
        const int s = x / (D * D / 8), rem = x % (D * D / 8), c = rem / (D / 8), f8 = rem % (D / 8);
        const int g = c / (D / 4), ci = c % (D / 4), row = 16 * (ci / 4) + 4 * g + ci % 4;
        *reinterpret_cast<uint4 *>(&sxy[s][row][8 * f8]) =
            *reinterpret_cast<const uint4 *>(xt + static_cast<size_t>(s) * D * D + static_cast<size_t>(c) * D + 8 * f8);
    }
    if (ROPE && tid < D / 2) rev[tid] = rope_rev_per_pos(tid, D, p.rope_base);
    lds_barrier();
    const float invN = 1.f / static_cast<float>(N);
    // one step: take the queries held in x, load step st + 2 into x, then the outputs (skipped when
    // the step lies past the sequence)
    auto step = [&](Qs &x, const int st) __attribute__((always_inline)) {
        const int tb0 = t0 + 16 * (wv + NW * st);
        const Qs c = x;
        load(x, st + 2);
        if (tb0 >= N) return;
        const int t = tb0 + l16;
        const bool ok = t < N;
        uint4 cq[KS];
        float ss = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint32_t wq[4] = {c.q[ks].x, c.q[ks].y, c.q[ks].z, c.q[ks].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = dot2_bf16(wq[i], ss);
            if (ROPE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // the pair (2j, 2j+1) sits in one 32-bit word: j = 16 ks + 4 g4 + i
                    float cs, sn;
                    rope_cos_sin(rev[16 * ks + 4 * g4 + i], t, cs, sn);
                    const float a = lo_f(wq[i]), b = hi_f(wq[i]);
                    wq[i] = pack2(a * cs - b * sn, a * sn + b * cs);
                }
            }
            cq[ks] = make_uint4(wq[0], wq[1], wq[2], wq[3]);
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        const float iq = ok ? __frsqrt_rn(fmaxf(ss, 1e-24f)) : 0.f;
        const float s1 = ok ? __fdividef(1.f, 1.f + __expf(-lo_f(c.g1))) : 0.f;
        const float sh = ok ? __fdividef(1.f, 1.f + __expf(-lo_f(c.gh))) : 0.f;
        const float ax = sh * iq, ay = (s1 - sh) * invN * iq;
        const float ah = (NS == 3 && ok) ? __fdividef(1.f, 1.f + __expf(-lo_f(c.g0))) * invN * iq : 0.f;
        uint32_t ow[D / 8];    // columns (D/4) g4 + [0, D/4) of token t, packed
#pragma unroll
        for (int ct = 0; ct < NFT; ++ct) {
            f32x4 accX = {0.f, 0.f, 0.f, 0.f}, accY = accX, accH = accX;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 B = as_bf16x8(cq[ks].x, cq[ks].y, cq[ks].z, cq[ks].w);
                const int f0 = 32 * ks + 8 * g4;
                accX = mfma(*reinterpret_cast<const bf16x8 *>(&sxy[0][16 * ct + l16][f0]), B, accX);
                accY = mfma(*reinterpret_cast<const bf16x8 *>(&sxy[1][16 * ct + l16][f0]), B, accY);
                if (NS == 3) accH = mfma(*reinterpret_cast<const bf16x8 *>(&sxy[NS - 1][16 * ct + l16][f0]), B, accH);
            }
            float r4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) r4[i] = ax * accX[i] + ay * accY[i] + (NS == 3 ? ah * accH[i] : 0.f);
            ow[2 * ct] = pack2(r4[0], r4[1]);
            ow[2 * ct + 1] = pack2(r4[2], r4[3]);
        }
        if (ok) {
            uint16_t *orow = o + static_cast<size_t>(t) * D + (D / 4) * g4;
#pragma unroll
            for (int j = 0; j < D / 32; ++j)
                *reinterpret_cast<uint4 *>(orow + 8 * j) = make_uint4(ow[4 * j], ow[4 * j + 1], ow[4 * j + 2], ow[4 * j + 3]);
        }
    };
    static_assert(SPW % 2 == 0, "steps per wave");
    for (int st = 0; st < SPW; st += 2) {
        step(qs0, st);
        step(qs1, st + 1);
    }
}

template <int D, bool ROPE, int NS>
hipError_t launch_v(const Problem &p, const LongWork &w, hipStream_t stream) {
    const int bh = p.B * p.H;
    hipLaunchKernelGGL((enc_long_logits_kernel<D>), dim3(bh * w.nsb), dim3(kLThreads), 0, stream, p, w);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((enc_long_state_kernel<D, ROPE, NS>), dim3(bh * w.nsb), dim3(kv_threads<D>()), 0, stream, p, w);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(enc_long_reduce_kernel, dim3(bh, (NS * D * D / 4 + 255) / 256), dim3(256), 0, stream, w, D * D, NS);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int nob = (p.N + out_block<D>() - 1) / out_block<D>();
    hipLaunchKernelGGL((enc_long_out_kernel<D, ROPE, NS>), dim3(bh * nob), dim3(out_threads<D>()), 0, stream, p, w);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem &p, const LongWork &w, hipStream_t stream) {
    const bool g0 = p.g0 != nullptr;
    if (p.rope) return g0 ? launch_v<D, true, 3>(p, w, stream) : launch_v<D, true, 2>(p, w, stream);
    return g0 ? launch_v<D, false, 3>(p, w, stream) : launch_v<D, false, 2>(p, w, stream);
}

}  // namespace

size_t encoder_long_work_bytes(const Problem &p) {
    const Sizes z = sizes(p, long_plan(p));
    return z.usum + z.s + z.aggb + z.xpart + z.xt;
}

hipError_t launch_encoder_long(const Problem &p, void *work, hipStream_t stream) {
    if (work == nullptr || p.N <= 0) return hipErrorInvalidValue;
    const LongWork w = carve(work, p);
    hipError_t err = launch_usum(p, w.usum, stream);
    if (err != hipSuccess) return err;
    switch (p.d) {
        case 64: return launch_d<64>(p, w, stream);
        case 128: return launch_d<128>(p, w, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zeros
