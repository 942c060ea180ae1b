// Causal ZeroS forward, float32 path (all d, both storage types): float32 arithmetic throughout,
// the contractions on the float32 matrix cores (v_mfma_f32_16x16x4f32), the rest on the vector ALU.
//
// Method: Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers",
// 关键设计 (zero-sum weights, radial-angular decoupling, deviation logits, linear-time prefix
// scan). Per head the output is o_t = sum_{i<=t} (alpha_t e^{s_i} + beta_t s_i + gamma_t)
// (q^_t . k^_i) v_i, which the prefix states turn into a recurrence; the optional zero-order gate
// of the same section adds sigma0_t / t to gamma_t.
//
// Work split: one workgroup per (batch, head, 16-column tile of v/o). The workgroup walks the
// sequence in chunks of kC tokens. For a chunk covering (t0, t1]:
//   o_t = sum_{t0<i<=t} W_{t,i} v_i + q^_t (a_t e^{m0-m_t} F + beta_t G + gamma_t H)   (states at t0)
// with W_{t,i} = (q^_t.k^_i)(a_t e^{s_i-m_t} + beta_t s_i + gamma_t), a_t = sigmah_t / E_t, and
// E, F rescaled by the running logit maximum m. The chunk then folds its keys into F, G, H.
// The states live in LDS (float32); K Q^T, the output products and the fold are 16x16 tiles per wave.
// The logits s_i and the per-segment u sums come from logits.hip (computed once per head, ahead of
// this kernel); the scalar scans are recomputed by every tile of a head (O(C) per chunk).
// A continued sequence (state in: the recurrence of the linear-time prefix scan paused after
// t_in tokens) starts from that state's F, G, H, m, E, P, with positions shifted by t_in.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace zeros {
namespace {

constexpr int kC = 32;         // tokens per chunk (64 measured no faster)
constexpr int kThreads = 256;  // 4 waves
constexpr int kTile = 16;      // value columns per workgroup
constexpr int kCPT = kTile / 8;  // value columns per thread in the staging and output passes
constexpr int kTPR = 8;        // threads per token row in the load phase

template <int D>
struct CausalSmem {
    float qh[kC][D + 1];   // normalised (and rotated) queries of the chunk
    float kh[kC][D + 1];   // normalised (and rotated) keys
    float vt[kC][kTile];   // this workgroup's value columns
    float W[kC][kC + 1];   // intra-chunk weights times cosines
    float F[D][kTile], G[D][kTile], Hs[D][kTile];
    float part[4][kC][kTile];  // the output pass's four products (q^ F, q^ G, q^ H scaled; W V)
    float s[kC], sig1[kC], sigh[kC], sig0[kC];   // sig0: zero-order gate (0 when off)
    float a_in[kC];        // a_t e^{m0 - m_t}: multiplies the carried F
    float a_loc[kC];       // a_t = sigmah_t / E_t (E relative to m_t)
    float mrow[kC], brow[kC], grow[kC];
    float estate[kC];      // e^{s_i - m1}: key weight of the F update
    float carry[4];        // m1, E1, P1 at the chunk end and the decay e^{m0 - m1}
};

template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i) { return to_f32(p[i]); }

// One launch runs either pass 1 (pass1 = 1: segments 0 .. nseg-2 from a zero state, writing their
// local sums and the logit maximum at their end, no outputs) or the main pass (every segment from
// its start state: outputs, and the final state in the last segment). With nseg = 1 the main pass
// is the whole sequence.
template <int D, typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void causal_valu_kernel(Problem p, ValuWork w, int nls, int pass1) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    CausalSmem<D> &sm = *reinterpret_cast<CausalSmem<D> *>(smem_raw);
    constexpr int NTILE = D / kTile;
    constexpr int EPT = D / kTPR;
    const int tid = threadIdx.x;

    // The NTILE workgroups of one head read the same q/k/u rows: keep them on one XCD
    // (consecutive dispatch slots go round-robin over the 8 XCDs).
    const int G = gridDim.x;
    int L = blockIdx.x;
    if ((G & 7) == 0) L = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int nsg = pass1 ? w.nseg - 1 : w.nseg;   // segments this launch covers
    const int tile = L % NTILE;
    const int seg = (L / NTILE) % nsg;
    const int bh = (L / NTILE) / nsg;
    const int N = p.N;
    const int t_beg = seg * w.seg_chunks * kC, t_end = min(N, (seg + 1) * w.seg_chunks * kC);
    const float *useg = w.useg;
    const size_t row0 = static_cast<size_t>(bh) * N;
    const T *q = static_cast<const T *>(p.q) + row0 * D;
    const T *k = static_cast<const T *>(p.k) + row0 * D;
    const T *v = static_cast<const T *>(p.v) + row0 * D;
    const T *g1 = static_cast<const T *>(p.g1) + row0;
    const T *gh = static_cast<const T *>(p.gh) + row0;
    const T *g0 = p.g0 != nullptr ? static_cast<const T *>(p.g0) + row0 : nullptr;
    T *o = static_cast<T *>(p.o) + row0 * D;

    const float *srow = w.s + row0;
    // a continued sequence starts from the given state: its tokens are positions tin + 1 ...
    const bool cont = p.sin.F != nullptr;
    const int tin = cont ? p.sin.t[bh] : 0;

    const int lr = tid / kTPR, lp = tid % kTPR, c0 = lp * EPT;
    double rope_rev[ROPE ? EPT / 2 : 1];
    if (ROPE) {
#pragma unroll
        for (int jj = 0; jj < EPT / 2; ++jj) rope_rev[jj] = rope_rev_per_pos(c0 / 2 + jj, D, p.rope_base);
    }

    float m_c = cont ? p.sin.m[bh] : kNegInf, E_c = cont ? p.sin.E[bh] : 0.f, P_c = cont ? p.sin.P[bh] : 0.f;
    if (seg > 0) {
        // logit carry at the segment start: the state's plus the aggregates of the 64-token blocks
        // before it (segments start on block boundaries)
        if (tid < 64) {
            float m = tid == 0 ? m_c : kNegInf, e = tid == 0 ? E_c : 0.f, ps = tid == 0 ? P_c : 0.f;
            auto merge = [](float &ma, float &ea, const float mb, const float eb) {
                const float mx = fmaxf(ma, mb);
                ea = exp_diff(ma, mx) * ea + exp_diff(mb, mx) * eb;
                ma = mx;
            };
            const float4 *ag = w.agg + static_cast<size_t>(bh) * ((N + 63) / 64);
            for (int j = tid; j < t_beg / 64; j += 64) {
                const float4 a = ag[j];
                merge(m, e, a.x, a.y);
                ps += a.z;
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float m2 = __shfl_xor(m, off, 64), e2 = __shfl_xor(e, off, 64);
                ps += __shfl_xor(ps, off, 64);
                merge(m, e, m2, e2);
            }
            if (tid == 0) {
                sm.carry[0] = m;
                sm.carry[1] = e;
                sm.carry[2] = ps;
            }
        }
        __syncthreads();
        m_c = sm.carry[0];
        E_c = sm.carry[1];
        P_c = sm.carry[2];
        __syncthreads();          // sm.carry is written again by the first chunk's scan
    }

    // start state: the given one (first segment), the combined start state (later segments of the
    // main pass) or zero (pass 1)
    const size_t mat0 = static_cast<size_t>(bh) * D * D;
    const float *S0F = nullptr, *S0G = nullptr, *S0H = nullptr;
    size_t s0base = mat0;
    if (!pass1 && seg > 0) {
        const float *st = w.segst + (static_cast<size_t>(bh) * (w.nseg - 1) + seg - 1) * 3 * D * D;
        S0F = st;
        S0G = st + D * D;
        S0H = st + 2 * D * D;
        s0base = 0;
    } else if (!pass1 && cont) {
        S0F = p.sin.F;
        S0G = p.sin.G;
        S0H = p.sin.Hs;
    }
    for (int x = tid; x < D * kTile; x += kThreads) {
        const size_t idx = s0base + static_cast<size_t>(x / kTile) * D + tile * kTile + x % kTile;
        (&sm.F[0][0])[x] = S0F != nullptr ? S0F[idx] : 0.f;
        (&sm.G[0][0])[x] = S0F != nullptr ? S0G[idx] : 0.f;
        (&sm.Hs[0][0])[x] = S0F != nullptr ? S0H[idx] : 0.f;
    }

    // the rows of the next chunk are read while the current one is processed; a thread takes rows
    // lr + RSTEP rs (rs < RS) of the chunk
    constexpr int RSTEP = kThreads / kTPR, RS = kC / RSTEP;
    static_assert(kC % RSTEP == 0 && kThreads / 8 == RSTEP, "row split");
    const int vr = tid / 8, vm = (tid % 8) * kCPT;
    float nq[RS][EPT], nk[RS][EPT], nv[RS][kCPT], ng1 = 0.f, ngh = 0.f, ng0 = 0.f, ns = 0.f;
    auto prefetch = [&](const int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            const int tok = min(t0 + lr + RSTEP * rs, N - 1);   // in bounds; rows past N are zeroed below
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                const size_t idx = static_cast<size_t>(tok) * D + c0 + c;
                nq[rs][c] = ld(q, idx);
                nk[rs][c] = ld(k, idx);
            }
            const size_t vidx = static_cast<size_t>(min(t0 + vr + RSTEP * rs, N - 1)) * D + tile * kTile + vm;
#pragma unroll
            for (int c = 0; c < kCPT; ++c) nv[rs][c] = ld(v, vidx + c);
        }
        if (tid < kC) {
            ng1 = ld(g1, min(t0 + tid, N - 1));
            ngh = ld(gh, min(t0 + tid, N - 1));
            if (g0 != nullptr) ng0 = ld(g0, min(t0 + tid, N - 1));
            ns = srow[min(t0 + tid, N - 1)];
        }
    };
    if (t_beg < t_end) prefetch(t_beg);

    for (int t0 = t_beg; t0 < t_end; t0 += kC) {
        const int nval = min(kC, N - t0);

        // ---- normalise, rotate and stage the rows read ahead; read the next chunk's rows
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            const int lrr = lr + RSTEP * rs;
            const int tok = tin + t0 + lrr;      // 0-based position in the sequence (RoPE)
            const bool valid = lrr < nval;
            float xq[EPT], xk[EPT];
            float ssq = 0.f, ssk = 0.f;
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                xq[c] = valid ? nq[rs][c] : 0.f;
                xk[c] = valid ? nk[rs][c] : 0.f;
                ssq += xq[c] * xq[c];
                ssk += xk[c] * xk[c];
            }
            ssq = group_sum<kTPR>(ssq);
            ssk = group_sum<kTPR>(ssk);
            const float iq = 1.f / fmaxf(sqrtf(ssq), 1e-12f);
            const float ik = 1.f / fmaxf(sqrtf(ssk), 1e-12f);
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                xq[c] *= iq;
                xk[c] *= ik;
            }
            if (ROPE) {
#pragma unroll
                for (int jj = 0; jj < EPT / 2; ++jj) {
                    float cs, sn;
                    rope_cos_sin(rope_rev[jj], tok, cs, sn);
                    const float q0 = xq[2 * jj], q1 = xq[2 * jj + 1];
                    const float k0 = xk[2 * jj], k1 = xk[2 * jj + 1];
                    xq[2 * jj] = q0 * cs - q1 * sn;
                    xq[2 * jj + 1] = q0 * sn + q1 * cs;
                    xk[2 * jj] = k0 * cs - k1 * sn;
                    xk[2 * jj + 1] = k0 * sn + k1 * cs;
                }
            }
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                sm.qh[lrr][c0 + c] = xq[c];
                sm.kh[lrr][c0 + c] = xk[c];
            }
        }
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            const int vrr = vr + RSTEP * rs;
            const bool valid = vrr < nval;
#pragma unroll
            for (int c = 0; c < kCPT; ++c) sm.vt[vrr][vm + c] = valid ? nv[rs][c] : 0.f;
        }
        if (tid < kC) {
            const bool valid = tid < nval;
            sm.sig1[tid] = valid ? sigmoidf(ng1) : 0.f;
            sm.sigh[tid] = valid ? sigmoidf(ngh) : 0.f;
            sm.sig0[tid] = (valid && g0 != nullptr) ? sigmoidf(ng0) : 0.f;
            sm.s[tid] = valid ? ns : 0.f;
        }
        if (t0 + kC < t_end) prefetch(t0 + kC);
        lds_barrier();

        // ---- scans of (max, sum e^{s-max}, sum s) over the chunk, joined with the carry
        // (one wave, lane r = token t0 + r + 1). Sums of s and the running maximum are DPP prefix
        // scans; the sums of e^{s} take a causal fixed reference (the carried maximum, or the chunk's
        // first logit at the start of the sequence), one exponential per token. A lane whose running
        // maximum exceeds the reference by more than 60 takes the exact (max, sum) scan instead,
        // which is only formed when some lane needs it. Every lane's result depends on its own
        // prefix only, so outputs never depend on later tokens, not even in rounding.
        if (tid < 64) {
            const int r = tid;
            const bool valid = r < nval;
            const float sr = valid ? sm.s[r] : 0.f;
            const float ps = wave_scan_add(sr);
            const float mloc = wave_scan_max(valid ? sr : kNegInf);
            const float M = fmaxf(m_c, mloc);                      // m_t
            const float ref = (m_c == kNegInf) ? lane_f(sr, 0) : m_c;
            const bool fixed_ok = M - ref <= 60.f;
            const float pe = wave_scan_add(valid && fixed_ok ? expf(sr - ref) : 0.f);
            float E = (exp_diff(m_c, ref) * E_c + pe) * expf(ref - M);
            if (__builtin_amdgcn_ballot_w64(valid && !fixed_ok) != 0) {   // the same on every lane
                float m = valid ? sr : kNegInf, e = valid ? 1.f : 0.f;
#pragma unroll
                for (int off = 1; off < kC; off <<= 1) {
                    const float m2 = __shfl_up(m, off, 64);
                    const float e2 = __shfl_up(e, off, 64);
                    if (r >= off) {
                        const float Mx = fmaxf(m, m2);
                        e = e * exp_diff(m, Mx) + e2 * exp_diff(m2, Mx);
                        m = Mx;
                    }
                }
                if (!fixed_ok) E = E_c * exp_diff(m_c, M) + e * exp_diff(m, M);
            }
            const float P = P_c + ps;
            if (valid) {
                const float tt = static_cast<float>(tin + t0 + r + 1);
                const float s1 = sm.sig1[r], sh = sm.sigh[r];
                const float a = sh / E;
                const float d1 = s1 - sh;
                sm.a_loc[r] = a;
                sm.a_in[r] = a * exp_diff(m_c, M);
                sm.mrow[r] = M;
                sm.brow[r] = d1 / tt;
                // the zero-order term adds sigma0_t / t to gamma
                sm.grow[r] = -d1 * (P / tt) / tt + (sm.sig0[r] - sh) / tt;
            }
            if (r == nval - 1) {
                sm.carry[0] = M;
                sm.carry[1] = E;
                sm.carry[2] = P;
                sm.carry[3] = exp_diff(m_c, M);
            }
        }
        lds_barrier();
        const float m_new = sm.carry[0];
        if (tid < kC) sm.estate[tid] = (tid < nval) ? expf(sm.s[tid] - m_new) : 0.f;
        if (pass1) {
            lds_barrier();      // key weights visible to the fold; pass 1 forms no outputs
        } else {

        // ---- intra-chunk weights W_{t,i} (i <= t): A^T = K Q^T on the float32 matrix cores, the 16x16
        // tiles (key tile kt, query tile qt) taken by the waves in turn (A[key][f] = k^[key][f],
        // B[f][query] = q^[query][f]); the accumulator lane holds keys 16 kt + 4 g4 + [0, 4) of query
        // 16 qt + l16. Tiles with every key after every query are zero.
        {
            static_assert(kThreads / 64 == 4 && kC % 16 == 0 && kC <= 64, "intra-chunk pass shape");
            constexpr int NTT = kC / 16;                     // 16-token tiles per chunk
            const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l16 = lane & 15, g4 = lane >> 4;
            for (int ti = wv; ti < NTT * NTT; ti += 4) {     // tiles (kt, qt) in turn over the waves
                const int kt = ti % NTT, qt = ti / NTT;
                const int t = 16 * qt + l16;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (kt <= qt) {
#pragma unroll 4
                    for (int k0 = 0; k0 < D; k0 += 4)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.kh[16 * kt + l16][k0 + g4], sm.qh[t][k0 + g4], acc, 0, 0, 0);
                }
                const float at = sm.a_loc[t], mt = sm.mrow[t], bt = sm.brow[t], gt = sm.grow[t];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * kt + 4 * g4 + r;
                    float w = 0.f;
                    if (i <= t && t < nval) {
                        const float si = sm.s[i];
                        w = acc[r] * (at * expf(si - mt) + bt * si + gt);
                    }
                    sm.W[t][i] = w;
                }
            }
        }
        lds_barrier();

        // ---- outputs on the float32 matrix cores: wave 0, 1, 2 forms q^ F, q^ G, q^ H (scaled per token
        // by a_in, beta, gamma), wave 3 the intra-chunk W V, each for both 16-token tiles; the
        // products meet in LDS. Tile (columns l16 ... as A rows, tokens as B columns):
        //   q^ S: A[col][f] = S[f][col], B[f][tok] = q^[tok][f];   W V: A[col][i] = v[i][col], B[i][tok] = W[tok][i]
        // and the accumulator lane holds columns 4 g4 + [0, 4) of token 16 tt + l16.
        {
            static_assert(kThreads / 64 == 4 && kTile == 16 && kC % 16 == 0, "output pass shape");
            const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
            for (int tt = 0; tt < kC / 16; ++tt) {
                const int tok = 16 * tt + l16;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (wv < 3) {
                    const float(*S)[kTile] = wv == 0 ? sm.F : (wv == 1 ? sm.G : sm.Hs);
#pragma unroll 4
                    for (int k0 = 0; k0 < D; k0 += 4)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(S[k0 + g4][l16], sm.qh[tok][k0 + g4], acc, 0, 0, 0);
                    const float cf = wv == 0 ? sm.a_in[tok] : (wv == 1 ? sm.brow[tok] : sm.grow[tok]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] *= cf;
                } else {
#pragma unroll
                    for (int k0 = 0; k0 < kC; k0 += 4)       // W[t][i] = 0 for i > t
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.vt[k0 + g4][l16], sm.W[tok][k0 + g4], acc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.part[wv][tok][4 * g4 + i] = acc[i];
            }
        }
        lds_barrier();
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            const int t = tid / 8 + RSTEP * rs, m0 = (tid % 8) * kCPT;
            if (t < nval) {
                const size_t idx = static_cast<size_t>(t0 + t) * D + tile * kTile + m0;
#pragma unroll
                for (int c = 0; c < kCPT; ++c) {
                    const float out = (sm.part[0][t][m0 + c] + sm.part[1][t][m0 + c]) +
                                      (sm.part[2][t][m0 + c] + sm.part[3][t][m0 + c]);
                    o[idx + c] = from_f32<T>(out);
                }
            }
        }
        // (no barrier: the fold reads the staged rows and writes F, G, H, which the output products
        // finished reading before the barrier above; the products in LDS are not touched again
        // before the barrier at the end of the chunk)
        }

        // ---- fold the chunk's keys into the states on the float32 matrix cores (exact float32
        // products, float32 sums): wave w owns 16-row tiles rt = w, w + 4, ... of F, G, H.
        // A = k^T (rows: features 16 rt + l16, k: keys k0 + g4), B = the weighted v (k: keys, columns
        // l16); the accumulator lane holds rows 16 rt + 4 g4 + [0, 4) of column l16.
        {
            const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l16 = lane & 15, g4 = lane >> 4;
            const float decay = sm.carry[3];
            for (int rt = wv; rt < D / 16; rt += kThreads / 64) {
                f32x4 aF, aG, aH;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = 16 * rt + 4 * g4 + i;
                    aF[i] = decay * sm.F[j][l16];
                    aG[i] = sm.G[j][l16];
                    aH[i] = sm.Hs[j][l16];
                }
#pragma unroll
                for (int k0 = 0; k0 < kC; k0 += 4) {         // absent keys: k^ and v rows are zero
                    const int key = k0 + g4;
                    const float a = sm.kh[key][16 * rt + l16];
                    const float vv = sm.vt[key][l16];
                    aF = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sm.estate[key] * vv, aF, 0, 0, 0);
                    aG = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sm.s[key] * vv, aG, 0, 0, 0);
                    aH = __builtin_amdgcn_mfma_f32_16x16x4f32(a, vv, aH, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = 16 * rt + 4 * g4 + i;
                    sm.F[j][l16] = aF[i];
                    sm.G[j][l16] = aG[i];
                    sm.Hs[j][l16] = aH[i];
                }
            }
        }
        m_c = m_new;
        E_c = sm.carry[1];
        P_c = sm.carry[2];
        lds_barrier();
    }

    if (pass1) {
        // segment-local sums (F relative to the logit maximum at the segment end) for the combine
        float *dst = w.segst + (static_cast<size_t>(bh) * (w.nseg - 1) + seg) * 3 * D * D;
        for (int x = tid; x < D * kTile; x += kThreads) {
            const size_t idx = static_cast<size_t>(x / kTile) * D + tile * kTile + x % kTile;
            dst[idx] = (&sm.F[0][0])[x];
            dst[D * D + idx] = (&sm.G[0][0])[x];
            dst[2 * D * D + idx] = (&sm.Hs[0][0])[x];
        }
        if (tile == 0 && tid == 0) w.segm[static_cast<size_t>(bh) * w.nseg + seg] = m_c;
        return;
    }

    // ---- final state
    if (p.st.F != nullptr && seg == w.nseg - 1) {
        for (int x = tid; x < D * kTile; x += kThreads) {
            const int j = x / kTile, mm = x % kTile;
            const size_t idx = mat0 + static_cast<size_t>(j) * D + tile * kTile + mm;
            p.st.F[idx] = sm.F[j][mm];
            p.st.G[idx] = sm.G[j][mm];
            p.st.Hs[idx] = sm.Hs[j][mm];
        }
        if (tile == 0) {
            if (tid < D) {
                float su = cont ? p.sin.Su[static_cast<size_t>(bh) * D + tid] : 0.f;
                for (int sg = 0; sg < nls; ++sg) su += useg[(static_cast<size_t>(bh) * nls + sg) * D + tid];
                p.st.Su[static_cast<size_t>(bh) * D + tid] = su;
            }
            if (tid == 0) {
                p.st.m[bh] = m_c;
                p.st.E[bh] = E_c;
                p.st.P[bh] = P_c;
                p.st.t[bh] = tin + N;
            }
        }
    }
}

// Start states of segments 1 .. nseg-1, one element of the d x d matrices per thread, in place over
// the segment-local sums: F <- e^{m_prev - m_end} F + L_F, G <- G + L_G, H <- H + L_H per segment,
// from the given state (continued sequence) or zero.
// Block (bh, 0) also writes the logit carry (m, E, P) at the start of every segment: the given
// state's merged with the (max, sum e^{s - max}, sum s) aggregates of the 64-token blocks before
// the segment, as an in-order lane scan over the blocks.
template <int D>
__global__ __launch_bounds__(256) void causal_valu_combine_kernel(Problem p, ValuWork w) {
    const int bh = blockIdx.x;
    const bool cont = p.sin.F != nullptr;
    if (blockIdx.y == 0 && threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int bps = w.seg_chunks / 2;                 // 64-token blocks per segment
        const int nb = (w.nseg - 1) * bps;                // blocks before the last segment
        const float4 *ag = w.agg + static_cast<size_t>(bh) * ((p.N + 63) / 64);
        float4 *sc = w.segc + static_cast<size_t>(bh) * w.nseg;
        float cm = cont ? p.sin.m[bh] : kNegInf, ce = cont ? p.sin.E[bh] : 0.f, cp = cont ? p.sin.P[bh] : 0.f;
        if (lane == 0) sc[0] = make_float4(cm, ce, cp, 0.f);
        for (int b0 = 0; b0 < nb; b0 += 64) {
            float m = kNegInf, e = 0.f, ps = 0.f;
            if (b0 + lane < nb) {
                const float4 a = ag[b0 + lane];
                m = a.x;
                e = a.y;
                ps = a.z;
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float m2 = __shfl_up(m, off, 64), e2 = __shfl_up(e, off, 64), p2 = __shfl_up(ps, off, 64);
                if (lane >= off) {
                    const float mx = fmaxf(m2, m);
                    e = e2 * exp_diff(m2, mx) + e * exp_diff(m, mx);
                    m = mx;
                    ps = p2 + ps;
                }
            }
            const float mx = fmaxf(cm, m);
            const float E = ce * exp_diff(cm, mx) + e * exp_diff(m, mx), P = cp + ps;
            const int blk = b0 + lane;
            if (blk < nb && (blk + 1) % bps == 0) sc[(blk + 1) / bps] = make_float4(mx, E, P, 0.f);
            const int last = min(63, nb - 1 - b0);
            cm = lane_f(mx, last);
            ce = lane_f(E, last);
            cp = lane_f(P, last);
        }
    }
    const int x = blockIdx.y * blockDim.x + threadIdx.x;
    if (x >= D * D) return;
    const size_t e = static_cast<size_t>(bh) * D * D + x;
    float f = cont ? p.sin.F[e] : 0.f, g = cont ? p.sin.G[e] : 0.f, h = cont ? p.sin.Hs[e] : 0.f;
    float m = cont ? p.sin.m[bh] : kNegInf;
    // segments whose sums are loaded together: the loads are unconditional (the index clamped to the
    // last segment) so they issue back to back; a guard per load compiles to a branch and a wait each.
    // Batches of 4 segments when there are few, of 32 when there are many.
    auto chain = [&](auto batch) __attribute__((always_inline)) {
        constexpr int kBatch = decltype(batch)::value;
        for (int j0 = 0; j0 + 1 < w.nseg; j0 += kBatch) {
            const int nj = min(kBatch, w.nseg - 1 - j0);
            float lf[kBatch], lg[kBatch], lh[kBatch], lm[kBatch];
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                const int j = min(j0 + jj, w.nseg - 2);
                const float *st = w.segst + (static_cast<size_t>(bh) * (w.nseg - 1) + j) * 3 * D * D;
                lf[jj] = st[x];
                lg[jj] = st[D * D + x];
                lh[jj] = st[2 * D * D + x];
                lm[jj] = w.segm[static_cast<size_t>(bh) * w.nseg + j];
            }
#pragma unroll
            for (int jj = 0; jj < kBatch; ++jj) {
                if (jj < nj) {
                    float *st = w.segst + (static_cast<size_t>(bh) * (w.nseg - 1) + j0 + jj) * 3 * D * D;
                    f = exp_diff(m, lm[jj]) * f + lf[jj];
                    g += lg[jj];
                    h += lh[jj];
                    st[x] = f;
                    st[D * D + x] = g;
                    st[2 * D * D + x] = h;
                    m = lm[jj];
                }
            }
        }
    };
    if (w.nseg <= 5) chain(std::integral_constant<int, 4>{});
    else chain(std::integral_constant<int, 32>{});
}

template <int D, typename T, bool ROPE>
hipError_t launch_one(const Problem &p, const ValuWork &w, hipStream_t stream) {
    const size_t smem = sizeof(CausalSmem<D>);
    const void *fn = reinterpret_cast<const void *>(&causal_valu_kernel<D, T, ROPE>);
    hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(smem));
    if (err != hipSuccess) return err;
    const int grid = p.B * p.H * (D / kTile);
    const int nls = (p.N + kLogitSeg - 1) / kLogitSeg;
    if (w.nseg > 1) {
        hipLaunchKernelGGL((causal_valu_kernel<D, T, ROPE>), dim3(grid * (w.nseg - 1)), dim3(kThreads), smem,
                           stream, p, w, nls, 1);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if ((err = launch_valu_combine(p, w, stream)) != hipSuccess) return err;
    }
    hipLaunchKernelGGL((causal_valu_kernel<D, T, ROPE>), dim3(grid * w.nseg), dim3(kThreads), smem, stream, p, w,
                       nls, 0);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem &p, const ValuWork &w, hipStream_t stream) {
    if (p.dtype == ZEROS_BF16)
        return p.rope ? launch_one<D, bf16, true>(p, w, stream) : launch_one<D, bf16, false>(p, w, stream);
    return p.rope ? launch_one<D, float, true>(p, w, stream) : launch_one<D, float, false>(p, w, stream);
}

// workspace regions start on 256-byte boundaries
size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// Segments of the scan: whole 64-token blocks (an even number of chunks). The per-tile kernel (d 16
// and 32, and bfloat16 state copies) takes at least four chunks per segment and enough (head, tile,
// segment) workgroups for one per CU; a grid that already fills the chip is left whole (its chunk
// work is bound by the CUs' throughput: three workgroups per CU measured no faster than one). The
// per-head float32 kernel (d 64 and 128) takes enough (head, segment) workgroups for one per CU, at
// most kF32MaxSeg segments per head (the combine chains them in order).
constexpr int kF32MaxSeg = 64;
// The per-head kernel addresses one head's rows with 32-bit offsets.
bool f32_per_head(int d, int N) { return d >= 64 && static_cast<long long>(N) * d * 4 < (1LL << 31); }
void valu_seg_plan(int B, int H, int N, int d, int &nseg, int &seg_chunks) {
    const int nch = (N + kC - 1) / kC;
    const bool per_head = f32_per_head(d, N);
    const long wg = static_cast<long>(B) * H * (per_head ? 1 : d / kTile);
    long want = (256 + wg - 1) / wg;
    if (want > nch / (per_head ? 2 : 4)) want = nch / (per_head ? 2 : 4);
    if (per_head && want > kF32MaxSeg) want = kF32MaxSeg;
    if (want < 1) want = 1;
    seg_chunks = static_cast<int>((nch + want - 1) / want);
    seg_chunks += seg_chunks & 1;
    nseg = nch > 0 ? (nch + seg_chunks - 1) / seg_chunks : 1;
}

}  // namespace

// Workspace of the float32 / small-d causal path: logits [B H, N], u sums per logit segment
// [B H, nls, d_u], per-64-token logit aggregates [B H, ceil(N/64)] (written by the logits kernels),
// and for a segmented scan the segment states [B H, nseg-1, 3, d, d], maxima [B H, nseg] and the
// logit carries (m, E, P) at the segment starts [B H, nseg].
size_t causal_valu_work_bytes(int B, int H, int N, int du) {
    const size_t bh = static_cast<size_t>(B) * H;
    const size_t nls = (static_cast<size_t>(N) + kLogitSeg - 1) / kLogitSeg;
    const size_t n64 = (static_cast<size_t>(N) + 63) / 64;
    int nseg, seg_chunks;
    valu_seg_plan(B, H, N, du, nseg, seg_chunks);
    size_t b = up256(bh * N * 4) + up256(bh * nls * du * 4) + up256(bh * n64 * 16);
    if (nseg > 1) b += up256(bh * (nseg - 1) * size_t(3) * du * du * 4) + up256(bh * nseg * 4) + up256(bh * nseg * 16);
    return b;
}

ValuWork causal_valu_work_carve(void *base, int B, int H, int N, int du) {
    const size_t bh = static_cast<size_t>(B) * H;
    const size_t nls = (static_cast<size_t>(N) + kLogitSeg - 1) / kLogitSeg;
    const size_t n64 = (static_cast<size_t>(N) + 63) / 64;
    char *b = static_cast<char *>(base);
    ValuWork w{};
    valu_seg_plan(B, H, N, du, w.nseg, w.seg_chunks);
    w.s = reinterpret_cast<float *>(b);
    b += up256(bh * N * 4);
    w.useg = reinterpret_cast<float *>(b);
    b += up256(bh * nls * du * 4);
    w.agg = reinterpret_cast<float4 *>(b);
    b += up256(bh * n64 * 16);
    if (w.nseg > 1) {
        w.segst = reinterpret_cast<float *>(b);
        b += up256(bh * (w.nseg - 1) * size_t(3) * du * du * 4);
        w.segm = reinterpret_cast<float *>(b);
        b += up256(bh * w.nseg * 4);
        w.segc = reinterpret_cast<float4 *>(b);
    }
    return w;
}

hipError_t launch_valu_combine(const Problem &p, const ValuWork &w, hipStream_t stream) {
    // one thread per state element, each chaining all segments; with few heads, one-wave blocks
    // spread the chains over more CUs
    const int nt = p.B * p.H < 64 ? 64 : 256;
    const dim3 grid(p.B * p.H, (p.d * p.d + nt - 1) / nt);
    switch (p.d) {
        case 16: hipLaunchKernelGGL((causal_valu_combine_kernel<16>), grid, dim3(nt), 0, stream, p, w); break;
        case 32: hipLaunchKernelGGL((causal_valu_combine_kernel<32>), grid, dim3(nt), 0, stream, p, w); break;
        case 64: hipLaunchKernelGGL((causal_valu_combine_kernel<64>), grid, dim3(nt), 0, stream, p, w); break;
        case 128: hipLaunchKernelGGL((causal_valu_combine_kernel<128>), grid, dim3(nt), 0, stream, p, w); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_causal_valu(const Problem &p, const ValuWork &w, hipStream_t stream) {
    hipError_t err = launch_logits(p, w.useg, w.s, w.agg, stream);
    if (err != hipSuccess) return err;
    // float32 with d 64 or 128: the per-head kernel (a bfloat16 call reaches this path only as a copy
    // of the state with N = 0, which the per-tile kernel does)
    if (p.dtype == ZEROS_F32 && f32_per_head(p.d, p.N)) return launch_causal_f32(p, w, stream);
    switch (p.d) {
        case 16: return launch_d<16>(p, w, stream);
        case 32: return launch_d<32>(p, w, stream);
        case 64: return launch_d<64>(p, w, stream);
        case 128: return launch_d<128>(p, w, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zeros
