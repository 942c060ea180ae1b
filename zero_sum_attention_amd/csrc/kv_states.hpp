// Weighted key-value state sums on the matrix cores, over a token range of one head:
//   S_s += sum_i k^_i^T (v_i w_s(i))      (s = 0, 1: the weights w_X, w_Y of the caller; s = 2: 1)
// with k^ the unit key (optionally RoPE-rotated at its absolute position) and w_s computed per
// token from its logit. Used for the partial states of the encoder (Paper-Notes page "ZeroS:
// Zero-Sum Linear Attention for Efficient Transformers", 关键设计 with t = N) and for the
// segment-local states of the causal scan (the same sums over one segment, centred at its end).
//
// One workgroup of D/16 waves; wave w owns the 16-column tile w of every state and all its D/16
// feature tiles (accumulator lane (l16, g4) of tile ft: features 16 ft + 4 g4 + [0, 4), column
// 16 w + l16). Rounds of 64 tokens: the round's k^ and v w_s rows are staged token-major in LDS
// (one 16-byte store per row piece) and read as MFMA operands by transposing LDS reads, which order
// the contraction over the tokens as 32 ks + 4 g4 + [0, 4), then + 16 (the same for both operands).
// Two staging buffers: each wave stages round r + 1 interleaved with its products of round r, so the
// staging arithmetic runs while the matrix cores work, with one barrier per round. The rows of the
// next rounds are in flight meanwhile; loads of rounds past the range re-read its last round (from
// L2), so every load is unconditional.
#pragma once

#include "device_common.hpp"
#include "encoder_common.hpp"
#include "mfma_common.hpp"

namespace zeros {

// Row padding of the staging buffers (bf16 elements): the four rows that 16 lanes of a transposing
// read name must fall on disjoint banks (64 banks of 4 bytes): rows of 72 bf16 (36 words) and of
// 144 bf16 (72 words, 8 mod 64) do; 136 bf16 (68 words, 4 mod 64) would put two rows on 4 banks.
template <int D> constexpr int kv_pad() { return D == 64 ? 8 : 16; }

template <int D> constexpr int kv_threads() { return 64 * (D / 16); }
constexpr int kKvRound = 64;       // tokens per round

template <int D, int NS>
struct KvBuf {
    uint16_t kh[kKvRound][D + kv_pad<D>()];        // k^ rows of the round
    uint16_t vw[NS][kKvRound][D + kv_pad<D>()];    // v w_X, v w_Y (, v) rows
};
// two rounds: one staged while the other is on the matrix cores
template <int D, int NS>
struct KvSmem {
    KvBuf<D, NS> b[2];
};

template <int D, bool ROPE, int NS>
struct KvStates {
    static constexpr int NT = kv_threads<D>(), NW = NT / 64, RND = kKvRound;
    static constexpr int LPR = D / 8, RPP = NT / LPR, PPR = RND / RPP, NFT = D / 16;
    // each thread stages one row per 32-token step: row piece j of a round pairs with step ks = j
    static_assert(RPP == 32 && PPR * RPP == RND && NW == NFT, "state kernel shape");
    struct Rows {
        uint4 k[PPR], v[PPR];
        float s[PPR];
    };

    KvSmem<D, NS> &sm;
    const uint16_t *k, *v;     // the head's rows [N, D]
    const float *srow;         // the head's logits [N]
    const double *rev;         // RoPE revolutions per position of each pair (LDS), or null
    int N, t0, t1, nrd, pos0;  // tokens [t0, t1) of N; RoPE position of token r: pos0 + r
    int tid, lane, wv, l16, g4, fr, rr;
    Rows rows0, rows1;
    f32x4 acc[NS][NFT];

    __device__ __forceinline__ KvStates(KvSmem<D, NS> &sm_, const uint16_t *k_, const uint16_t *v_, const float *s_,
                                        const double *rev_, int N_, int t0_, int t1_, int pos0_)
        : sm(sm_), k(k_), v(v_), srow(s_), rev(rev_), N(N_), t0(t0_), t1(t1_), pos0(pos0_) {
        nrd = (t1 - t0 + RND - 1) / RND;
        tid = threadIdx.x;
        lane = tid & 63;
        wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        l16 = lane & 15;
        g4 = lane >> 4;
        fr = tid % LPR;
        rr = tid / LPR;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int i = 0; i < NFT; ++i) acc[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void load(Rows &x, int rd) {
        rd = min(rd, nrd - 1);
#pragma unroll
        for (int j = 0; j < PPR; ++j) {
            const int r = min(t0 + rd * RND + rr + RPP * j, N - 1);
            x.k[j] = *reinterpret_cast<const uint4 *>(k + static_cast<size_t>(r) * D + 8 * fr);
            x.v[j] = *reinterpret_cast<const uint4 *>(v + static_cast<size_t>(r) * D + 8 * fr);
            x.s[j] = srow[r];
        }
    }

    // the first two rounds in flight (before the caller's set-up, which ends with a barrier). The
    // loads of round 0 are issued before those of round 1, in the order of the loop's own loads, so
    // that the wait counts placed in the loop (loads complete in issue order) let the next round's
    // loads stay in flight while a round is staged.
    __device__ __forceinline__ void start() {
        load(rows0, 0);
        asm volatile("" ::: "memory");
        load(rows1, 1);
        asm volatile("" ::: "memory");
    }

    // transposing-read operand of 16-row tile `tile` of buffer b at 32-token step ks: lane (g4, l16)
    // names features 16 tile + 4 (l16 & 3) + [0, 4) of token 32 ks + 4 g4 + (l16 >> 2) (and + 16)
    __device__ __forceinline__ bf16x8 operand(const uint16_t (*b)[D + kv_pad<D>()], int tile, int ks) const {
        const int f = 16 * tile + 4 * (l16 & 3), r = 32 * ks + 4 * g4 + (l16 >> 2);
        const uint2 a = lds_tr16(&b[r][f]);
        const uint2 c = lds_tr16(&b[r + 16][f]);
        return as_bf16x8(a.x, a.y, c.x, c.y);
    }

    // RoPE phase of this thread's pairs 4 fr + [0, 4) at the start of round rd, in revolutions reduced
    // in double precision; a row adds its offset times the pair's rate and takes the hardware sine
    // and cosine of the fraction (as the causal main pass does)
    __device__ __forceinline__ void rope_base(int rd, float (&rbase)[4], float (&rrate)[4]) const {
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
            const double rv = rev[4 * fr + j2];
            const double b = static_cast<double>(pos0 + t0 + rd * RND) * rv;
            rbase[j2] = static_cast<float>(b - rint(b));
            rrate[j2] = static_cast<float>(rv);
        }
    }

    // row piece j of round rd (rows held in x) into buffer b: unit k^ (rotated) and v w_s; rows past
    // the range stage zeros
    template <class Weights>
    __device__ __forceinline__ void stage_row(const Rows &x, const int rd, const int j, KvBuf<D, NS> &b, const Weights &wfn,
                                              const float (&rbase)[4], const float (&rrate)[4]) const {
        const int rl = rr + RPP * j, r = t0 + rd * RND + rl;
        const bool ok = r < t1;
        float kv[8], vv[8];
        unpack8(x.k[j], kv);
        unpack8(x.v[j], vv);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(kv[i], kv[i], ss);
        ss = group_sum<LPR>(ss);
        const float ik = ok ? __frsqrt_rn(fmaxf(ss, 1e-24f)) : 0.f;
        if constexpr (ROPE) {
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                float ph = fmaf(static_cast<float>(rl), rrate[j2], rbase[j2]);
                ph -= rintf(ph);
                const float cs = __builtin_amdgcn_cosf(ph), sn = __builtin_amdgcn_sinf(ph);
                const float a = kv[2 * j2], c = kv[2 * j2 + 1];
                kv[2 * j2] = a * cs - c * sn;
                kv[2 * j2 + 1] = a * sn + c * cs;
            }
        }
        const float2 wt = wfn(x.s[j]);
        const float wx = ok ? wt.x : 0.f, wy = ok ? wt.y : 0.f;
        *reinterpret_cast<uint4 *>(&b.kh[rl][8 * fr]) = make_uint4(pack2(kv[0] * ik, kv[1] * ik), pack2(kv[2] * ik, kv[3] * ik),
                                                                   pack2(kv[4] * ik, kv[5] * ik), pack2(kv[6] * ik, kv[7] * ik));
        *reinterpret_cast<uint4 *>(&b.vw[0][rl][8 * fr]) = make_uint4(pack2(vv[0] * wx, vv[1] * wx), pack2(vv[2] * wx, vv[3] * wx),
                                                                      pack2(vv[4] * wx, vv[5] * wx), pack2(vv[6] * wx, vv[7] * wx));
        *reinterpret_cast<uint4 *>(&b.vw[1][rl][8 * fr]) = make_uint4(pack2(vv[0] * wy, vv[1] * wy), pack2(vv[2] * wy, vv[3] * wy),
                                                                      pack2(vv[4] * wy, vv[5] * wy), pack2(vv[6] * wy, vv[7] * wy));
        if constexpr (NS == 3)   // v itself (zero past the range)
            *reinterpret_cast<uint4 *>(&b.vw[NS - 1][rl][8 * fr]) = ok ? x.v[j] : make_uint4(0u, 0u, 0u, 0u);
    }

    // 32-token step ks of the round in buffer b on the matrix cores (rows past the range are zeros)
    __device__ __forceinline__ void products(const KvBuf<D, NS> &b, const int ks) {
        bf16x8 B[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) B[s] = operand(b.vw[s], wv, ks);
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            const bf16x8 A = operand(b.kh, ft, ks);
#pragma unroll
            for (int s = 0; s < NS; ++s) acc[s][ft] = mfma(A, B[s], acc[s][ft]);
        }
    }

    // one phase: stage round rd + 1 (rows in x) into buffer nb, step by step interleaved with the
    // products of round rd (buffer cb), then load round rd + 3 into x. One barrier per round: the
    // staged buffer was last read before the previous barrier.
    template <class Weights>
    __device__ __forceinline__ void phase(Rows &x, const int rd, const KvBuf<D, NS> &cb, KvBuf<D, NS> &nb, const Weights &wfn) {
        float rbase[4] = {0.f, 0.f, 0.f, 0.f}, rrate[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (ROPE) rope_base(rd + 1, rbase, rrate);
#pragma unroll
        for (int j = 0; j < PPR; ++j) {
            stage_row(x, rd + 1, j, nb, wfn, rbase, rrate);
            products(cb, j);
            // (one step's operands and staging values live at a time)
            if (j + 1 < PPR) asm volatile("" ::: "memory");
        }
        // (the next loads stay after this phase's work, so their registers are not held meanwhile)
        asm volatile("" ::: "memory");
        load(x, rd + 3);
        lds_barrier();
    }

    // all rounds; wfn(s) gives the (w_X, w_Y) weights of a token with logit s. Rounds past the range
    // (the last phase of an odd count) stage and multiply zeros.
    template <class Weights>
    __device__ __forceinline__ void run(const Weights &wfn) {
        {
            float rbase[4] = {0.f, 0.f, 0.f, 0.f}, rrate[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (ROPE) rope_base(0, rbase, rrate);
#pragma unroll
            for (int j = 0; j < PPR; ++j) stage_row(rows0, 0, j, sm.b[0], wfn, rbase, rrate);
            load(rows0, 2);
            lds_barrier();
        }
#pragma unroll 1
        for (int rd = 0; rd < nrd; rd += 2) {
            phase(rows1, rd, sm.b[0], sm.b[1], wfn);
            phase(rows0, rd + 1, sm.b[1], sm.b[0], wfn);
        }
    }
};

}  // namespace zeros
