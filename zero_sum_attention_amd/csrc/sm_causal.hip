// ZeroS-SM: the zero-sum reweighting of ZeroS applied to standard causal softmax attention, on the
// matrix cores (bfloat16 q, k, v with d in {64, 128}, float32 accumulation).
//
// Method: ai.info page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers", Methodology in
// Plain English (the same reweighting applied to standard softmax attention gives the quadratic-time
// variant ZeroS-SM); the split of a softmax row into its uniform, first-order and residual parts and
// the step gates follow the Paper-Notes page of the same title, 关键设计. With the logits
// l_{t,i} = q_t . k_i / sqrt(d) over the keys i <= t, their softmax p, their mean lbar_t and
// delta = l - lbar_t:
//   w_{t,i} = sigma1_t delta_{t,i} / t + sigmah_t (p_{t,i} - 1/t - delta_{t,i} / t)  (+ sigma0_t / t)
// so that, with A_t = sum p_{t,i} v_i, L_t = sum l_{t,i} v_i and V_t = sum_{i<=t} v_i,
//   o_t = sigmah_t A_t + ((sigma1_t - sigmah_t) / t) (L_t - lbar_t V_t) + ((sigma0_t - sigmah_t) / t) V_t.
// The three sums are accumulated together over blocks of 64 keys, A_t with the running maximum of
// an online softmax; lbar_t comes from the running sum of the logits.
//
// One workgroup of four waves per (batch, head, block of 64 queries); wave w owns the queries
// 16 w .. 16 w + 15 of the block. Per key block, staged in LDS (the K rows, and V transposed with its
// keys in the order below), each wave forms S^T = K Q^T (the block's keys by its 16 queries) on the
// matrix cores and then O^T += V^T P^T, V^T L^T and V^T M^T (M: the causal 0/1 mask). Their B operands
// come straight from the S^T accumulators: two 16-key tiles give a lane the keys {4 g4 + [0, 4)} and
// {16 + 4 g4 + [0, 4)} of a 32-key half, which is the order the keys of V^T are stored in.
// With RoPE, q and k are rotated once by a pass of their own into the caller's workspace.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace zeros {
namespace {

constexpr int kSmQ = 64;       // queries per workgroup (16 per wave)
constexpr int kSmK = 64;       // keys per block
constexpr int kSmPad = 8;      // bf16 elements of row padding in LDS

// Position of a key of a block along the contraction index of the output products (see above).
__device__ __forceinline__ int sm_kperm(int key) {
    return (key & ~31) | (((key & 15) >> 2) << 3) | (((key >> 4) & 1) << 2) | (key & 3);
}

__device__ __forceinline__ float bf16_bits_f32(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

struct SmArgs {
    const uint16_t *q, *k, *v, *g1, *gh, *g0;   // g0 NULL: no zero-order gate
    uint16_t *o;
    int N, BH, nqb;
};

template <int D>
__global__ __launch_bounds__(256, 2) void sm_causal_kernel(SmArgs a) {
    constexpr int KS = D / 32;                    // 32-feature steps of K Q^T
    constexpr int CTN = D / 16;                   // 16-column tiles of the output
    constexpr int KP = kSmK * (D / 8) / 256;      // 16-byte pieces of a K block per thread
    constexpr int VP = (kSmK / 2) * (D / 8) / 256;   // (key pair, 8-column group) items of a V block per thread
    static_assert(KP >= 1 && VP >= 1 && KP * 256 == kSmK * (D / 8) && VP * 256 == (kSmK / 2) * (D / 8),
                  "d must be 64 or 128");
    __shared__ __align__(16) uint16_t s_k[kSmK][D + kSmPad];
    __shared__ __align__(16) uint16_t s_vt[D][kSmK + kSmPad];
    __shared__ float s_vsum[D];                   // column sums of v over the full key blocks

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
    const int N = a.N;
    const int bh = static_cast<int>(blockIdx.x % a.BH);
    const int qb = a.nqb - 1 - static_cast<int>(blockIdx.x / a.BH);     // the longest rows first
    const size_t row0 = static_cast<size_t>(bh) * N;
    const uint16_t *kg = a.k + row0 * D, *vg = a.v + row0 * D;
    const int tq = qb * kSmQ + 16 * w + l16;      // this lane's query (0-based position)

    // Q^T as the B operand of K Q^T: features 32 ks + 8 g4 + [0, 8) of query tq (zero past N)
    bf16x8 bq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (tq < N) x = *reinterpret_cast<const uint4 *>(a.q + (row0 + tq) * D + 32 * ks + 8 * g4);
        bq[ks] = as_bf16x8(x.x, x.y, x.z, x.w);
    }

    // next key block in registers while the current one is in use; rows past N are zero
    uint4 pk[KP], pv[VP][2];
    auto fetch = [&](const int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int pc = tid + 256 * i, r = pc / (D / 8), c = pc % (D / 8), key = kb * kSmK + r;
            pk[i] = key < N ? *reinterpret_cast<const uint4 *>(kg + static_cast<size_t>(key) * D + 8 * c)
                            : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int it = tid + 256 * i, kp = it & 31, cg = it >> 5, key = kb * kSmK + 2 * kp;
            pv[i][0] = key < N ? *reinterpret_cast<const uint4 *>(vg + static_cast<size_t>(key) * D + 8 * cg)
                               : make_uint4(0u, 0u, 0u, 0u);
            pv[i][1] = key + 1 < N ? *reinterpret_cast<const uint4 *>(vg + static_cast<size_t>(key + 1) * D + 8 * cg)
                                   : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    // K rows as they are; V transposed, keys 2 kp and 2 kp + 1 of column m side by side at sm_kperm(2 kp)
    auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int pc = tid + 256 * i, r = pc / (D / 8), c = pc % (D / 8);
            *reinterpret_cast<uint4 *>(&s_k[r][8 * c]) = pk[i];
        }
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int it = tid + 256 * i, kp = it & 31, cg = it >> 5, pos = sm_kperm(2 * kp);
            const uint32_t x0[4] = {pv[i][0].x, pv[i][0].y, pv[i][0].z, pv[i][0].w};
            const uint32_t x1[4] = {pv[i][1].x, pv[i][1].y, pv[i][1].z, pv[i][1].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                *reinterpret_cast<uint32_t *>(&s_vt[8 * cg + 2 * j][pos]) = (x0[j] & 0xffffu) | (x1[j] << 16);
                *reinterpret_cast<uint32_t *>(&s_vt[8 * cg + 2 * j + 1][pos]) = (x0[j] >> 16) | (x1[j] & 0xffff0000u);
            }
        }
    };

    f32x4 ap[CTN], al[CTN];
#pragma unroll
    for (int ct = 0; ct < CTN; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) ap[ct][i] = al[ct][i] = 0.f;
    // running maximum of query tq's logits, and this lane's parts of sum e^{l - m} and sum l
    float m = kNegInf, lsum = 0.f, rsum = 0.f;
    const float rsd = 1.f / sqrtf(static_cast<float>(D));
    constexpr uint32_t kOne = 0x3f80u;            // bfloat16 1.0
    // V_t = sum_{i <= t} v_i: over the full key blocks (every key before every query of the
    // workgroup) a column sum, the same for all queries: thread = (column, part of the keys), its
    // sum over those blocks in vrun; over the diagonal block a product with the causal mask
    constexpr int VPARTS = 256 / D, VKEYS = kSmK / VPARTS;
    const int vcol = tid / VPARTS, vpart = tid % VPARTS;
    float vrun = 0.f;

    // one key block; DIAG: the block that holds this workgroup's queries (causal mask, and the mask
    // product for V_t)
    auto block = [&](const int kb, auto diag_c, f32x4 *a1) __attribute__((always_inline)) {
        constexpr bool DIAG = decltype(diag_c)::value;
        lds_barrier();                            // the previous block's LDS reads are done
        stage();
        lds_barrier();                            // this block is in LDS
        if (!DIAG) fetch(kb + 1);
        const bool diag = DIAG;
        // S^T = K Q^T: lane holds keys 16 kt + 4 g4 + i of query tq; in the diagonal block the
        // tiles whose keys all follow this wave's queries are skipped
        float lg[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (!diag || kt <= w) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(&s_k[16 * kt + l16][32 * ks + 8 * g4]);
                    acc = mfma(ak, bq[ks], acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) lg[kt][i] = acc[i] * rsd;
        }
        // causal mask (keys past tq: only in the diagonal block) and the online softmax
        const int key0 = kb * kSmK + 4 * g4;
        float mb = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key0 + 16 * kt + i <= tq) mb = fmaxf(mb, lg[kt][i]);
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float mn = fmaxf(m, mb);            // finite: key tq is in this block or an earlier one
        const float sc = (m == kNegInf) ? 0.f : __expf(m - mn);
#pragma unroll
        for (int ct = 0; ct < CTN; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) ap[ct][i] *= sc;
        lsum *= sc;
        m = mn;
        uint32_t pp[4][2], ll[4][2], mm[4][2] = {};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            float p4[4], l4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = key0 + 16 * kt + i <= tq;
                p4[i] = valid ? __expf(lg[kt][i] - mn) : 0.f;
                l4[i] = valid ? lg[kt][i] : 0.f;
                lsum += p4[i];
            }
            pp[kt][0] = pack2(p4[0], p4[1]);
            pp[kt][1] = pack2(p4[2], p4[3]);
            ll[kt][0] = pack2(l4[0], l4[1]);
            ll[kt][1] = pack2(l4[2], l4[3]);
            // the running sum of the logits takes the bfloat16 values of the L^T operand, so that the
            // first-order part sum (l - lbar) v keeps its zero sum over the keys exactly
            rsum += (lo_f(ll[kt][0]) + hi_f(ll[kt][0])) + (lo_f(ll[kt][1]) + hi_f(ll[kt][1]));
            if (DIAG) {
                const bool v0 = key0 + 16 * kt <= tq, v1 = key0 + 16 * kt + 1 <= tq;
                const bool v2 = key0 + 16 * kt + 2 <= tq, v3 = key0 + 16 * kt + 3 <= tq;
                mm[kt][0] = (v0 ? kOne : 0u) | (v1 ? kOne << 16 : 0u);
                mm[kt][1] = (v2 ? kOne : 0u) | (v3 ? kOne << 16 : 0u);
            }
        }
        // O^T += V^T P^T, V^T L^T (and V^T M^T in the diagonal block) over the two 32-key halves
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (diag && 32 * h > 16 * w + 15) continue;      // every key of the half follows the wave's queries
            const bf16x8 bp = as_bf16x8(pp[2 * h][0], pp[2 * h][1], pp[2 * h + 1][0], pp[2 * h + 1][1]);
            const bf16x8 bl = as_bf16x8(ll[2 * h][0], ll[2 * h][1], ll[2 * h + 1][0], ll[2 * h + 1][1]);
#pragma unroll
            for (int ct = 0; ct < CTN; ++ct) {
                const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&s_vt[16 * ct + l16][32 * h + 8 * g4]);
                ap[ct] = mfma(av, bp, ap[ct]);
                al[ct] = mfma(av, bl, al[ct]);
                if (DIAG) {
                    const bf16x8 bm = as_bf16x8(mm[2 * h][0], mm[2 * h][1], mm[2 * h + 1][0], mm[2 * h + 1][1]);
                    a1[ct] = mfma(av, bm, a1[ct]);
                }
            }
        }
        if (!DIAG) {
            // this thread's part of the column sum of the block (the keys' order does not matter)
#pragma unroll
            for (int j = 0; j < VKEYS / 8; ++j) {
                const uint4 x = *reinterpret_cast<const uint4 *>(&s_vt[vcol][VKEYS * vpart + 8 * j]);
                vrun += ((lo_f(x.x) + hi_f(x.x)) + (lo_f(x.y) + hi_f(x.y))) + ((lo_f(x.z) + hi_f(x.z)) + (lo_f(x.w) + hi_f(x.w)));
            }
        }
    };

    fetch(0);
    for (int kb = 0; kb < qb; ++kb) block(kb, std::false_type{}, nullptr);
    f32x4 a1[CTN];
#pragma unroll
    for (int ct = 0; ct < CTN; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) a1[ct][i] = 0.f;
    block(qb, std::true_type{}, a1);
    // the full blocks' column sums: the parts of a column are adjacent lanes
    vrun = group_sum<VPARTS>(vrun);
    if (vpart == 0) s_vsum[vcol] = vrun;
    lds_barrier();
#pragma unroll
    for (int ct = 0; ct < CTN; ++ct) {
        const float4 vs = *reinterpret_cast<const float4 *>(&s_vsum[16 * ct + 4 * g4]);
        a1[ct][0] += vs.x; a1[ct][1] += vs.y; a1[ct][2] += vs.z; a1[ct][3] += vs.w;
    }

    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    rsum += __shfl_xor(rsum, 16, 64);
    rsum += __shfl_xor(rsum, 32, 64);
    if (tq < N) {
        const size_t gi = row0 + tq;
        const float t1 = static_cast<float>(tq + 1);
        const float s1 = sigmoidf(bf16_bits_f32(a.g1[gi])), sh = sigmoidf(bf16_bits_f32(a.gh[gi]));
        const float s0 = a.g0 != nullptr ? sigmoidf(bf16_bits_f32(a.g0[gi])) : 0.f;
        const float ca = sh / lsum, c1 = (s1 - sh) / t1, lbar = rsum / t1, c0 = (s0 - sh) / t1;
#pragma unroll
        for (int ct = 0; ct < CTN; ++ct) {
            float r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r[i] = ca * ap[ct][i] + c1 * (al[ct][i] - lbar * a1[ct][i]) + c0 * a1[ct][i];
            // lane holds columns 16 ct + 4 g4 + [0, 4) of query tq
            *reinterpret_cast<uint2 *>(a.o + gi * D + 16 * ct + 4 * g4) = make_uint2(pack2(r[0], r[1]), pack2(r[2], r[3]));
        }
    }
}

// RoPE of standard attention: x (q or k, [rows, D] bfloat16, row r at position r % N) rotated by
// its position into y; pair j turns by position * base^(-2j/D), the angle reduced in revolutions in
// double precision before the hardware sine and cosine. Thread: 8 features (4 pairs) of one row.
template <int D>
__global__ __launch_bounds__(256) void sm_rope_kernel(const uint16_t *x, uint16_t *y, int N, size_t rows, float base) {
    __shared__ double s_rpp[D / 2];
    if (threadIdx.x < D / 2) s_rpp[threadIdx.x] = rope_rev_per_pos(threadIdx.x, D, base);
    __syncthreads();
    const size_t pc = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (pc >= rows * (D / 8)) return;
    const size_t row = pc / (D / 8);
    const int c = static_cast<int>(pc % (D / 8));
    const double pos = static_cast<double>(row % static_cast<size_t>(N));
    const uint4 in = *reinterpret_cast<const uint4 *>(x + row * D + 8 * c);
    const uint32_t wd[4] = {in.x, in.y, in.z, in.w};
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        double r = pos * s_rpp[4 * c + j];
        r -= rint(r);
        const float rev = static_cast<float>(r);
        const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
        const float x0 = lo_f(wd[j]), x1 = hi_f(wd[j]);
        out[j] = pack2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
    }
    *reinterpret_cast<uint4 *>(y + row * D + 8 * c) = make_uint4(out[0], out[1], out[2], out[3]);
}

template <int D>
hipError_t launch_sm_d(const Problem &p, void *work, hipStream_t stream) {
    const size_t rows = static_cast<size_t>(p.B) * p.H * p.N;
    const uint16_t *q = static_cast<const uint16_t *>(p.q), *k = static_cast<const uint16_t *>(p.k);
    if (p.rope) {
        uint16_t *qr = static_cast<uint16_t *>(work);
        uint16_t *kr = qr + rows * D;
        const unsigned grid = static_cast<unsigned>((rows * (D / 8) + 255) / 256);
        hipLaunchKernelGGL((sm_rope_kernel<D>), dim3(grid), dim3(256), 0, stream, q, qr, p.N, rows, p.rope_base);
        hipLaunchKernelGGL((sm_rope_kernel<D>), dim3(grid), dim3(256), 0, stream, k, kr, p.N, rows, p.rope_base);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        q = qr;
        k = kr;
    }
    SmArgs a;
    a.q = q;
    a.k = k;
    a.v = static_cast<const uint16_t *>(p.v);
    a.g1 = static_cast<const uint16_t *>(p.g1);
    a.gh = static_cast<const uint16_t *>(p.gh);
    a.g0 = static_cast<const uint16_t *>(p.g0);
    a.o = static_cast<uint16_t *>(p.o);
    a.N = p.N;
    a.BH = p.B * p.H;
    a.nqb = (p.N + kSmQ - 1) / kSmQ;
    hipLaunchKernelGGL((sm_causal_kernel<D>), dim3(a.BH * a.nqb), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t sm_work_bytes(const Problem &p) {
    if (!p.rope) return 0;
    return 2 * static_cast<size_t>(p.B) * p.H * p.N * p.d * 2;
}

hipError_t launch_sm_causal(const Problem &p, void *work, hipStream_t stream) {
    if (p.N == 0) return hipSuccess;
    if (p.d == 128) return launch_sm_d<128>(p, work, stream);
    if (p.d == 64) return launch_sm_d<64>(p, work, stream);
    return hipErrorInvalidValue;
}

}  // namespace zeros
