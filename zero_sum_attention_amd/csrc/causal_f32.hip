// Causal ZeroS forward, float32 inputs with d in {64, 128}: one workgroup per (batch, head,
// segment) with one wave per 16-column tile of v/o, float32 arithmetic throughout and every
// contraction on the float32 matrix cores (v_mfma_f32_16x16x4f32: exact float32 products, float32
// sums).
//
// Method: Paper-Notes page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers",
// 关键设计 (zero-sum weights, radial-angular decoupling, deviation logits, linear-time prefix
// scan). Per head o_t = sum_{i<=t} (alpha_t e^{s_i} + beta_t s_i + gamma_t) (q^_t . k^_i) v_i,
// carried by the prefix states F = sum e^{s_i - m} k^_i v_i^T (m the running logit maximum),
// G = sum s_i k^_i v_i^T and H = sum k^_i v_i^T; the optional zero-order gate adds sigma0_t / t to
// gamma_t.
//
// Chunks of C tokens (32 or 64); for a chunk covering (t0, t1]:
//   o_t = q^_t (a_t e^{m0 - m_t} F + beta_t G + gamma_t H) + sum_{t0<i<=t} W_{t,i} v_i   (states at t0)
//   W_{t,i} = (q^_t . k^_i)(a_t e^{s_i - m_t} + beta_t s_i + gamma_t),  a_t = sigmah_t / E_t,
// then F <- e^{m0 - m1} F + K^T diag(e^{s - m1}) V, G += K^T diag(s) V, H += K^T V.
//
// Layout. Wave w owns value columns [16w, 16w + 16) and holds its slice of F, G and H as matrix-core
// accumulators: lane (l, g) of 16-row tile r holds rows 16r + 4g + [0, 4) of column 16w + l. Those
// registers are directly the A operand of the output products q^ S, with the contraction index
// ordered to match (step (r, i) of lane group g takes feature 16r + 4g + i), so the states never
// leave the registers. The chunk's unit q^ and k^ rows are formed once per workgroup in LDS and
// shared by all tiles; the scalar scan of a chunk (max, sum e^{s - max}, sum s and the per-token
// coefficients) runs on the last wave one chunk ahead, after its share of the non-zero 16 x 16
// tiles of A^T = K Q^T and the weights W, which all waves form. Two barriers per chunk. The main pass skips the
// fold after its last chunk unless it writes the recurrent state.
//
// Long heads are cut into segments of whole 64-token blocks (pass 1: the states of segments
// 0 .. nseg-2 from zero, F relative to the running maximum at the segment end; a combine kernel
// chains them; the main pass runs every segment from its start state), so that B H nseg
// workgroups cover the chip.
#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace zeros {
namespace {

template <int D, int C, int RS>
struct F32Smem {
    static constexpr int NT = C / 16;   // 16-token tiles per chunk
    float qh[2][C][D + 4];      // unit (rotated) queries, by chunk parity
    float kh[2][C][D + 4];      // unit (rotated) keys
    float W[C][C + 4];          // intra-chunk weights times cosines, W[t][i] (i <= t)
    // per-token scan results by chunk parity: query-side coefficients and key weights
    float a_in[2][C];           // a_t e^{m0 - m_t}: multiplies the carried F
    float a_loc[2][C];          // a_t = sigmah_t / E_t (E relative to m_t)
    float mrow[2][C], brow[2][C], grow[2][C];
    float est[2][C];            // e^{s_i - m1}: key weight of the F update
    float s[2][C];              // logits (key weight of the G update)
    float decay[2];             // e^{m0 - m1}
    // row-split partial output products passed between the two waves of a column tile
    float4 xch[RS == 2 ? D / 16 : 1][RS == 2 ? NT : 1][64];
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// Buffer resource over n bytes at p (raw, dword data): loads take a 32-bit byte offset, and an
// offset at or past n reads zero instead of touching memory. Offsets are passed whole in the
// vector operand (the scalar offset stays 0) so every byte of the access is range-checked.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(n), 0x00020000);
}
// (the loads return raw 32-bit words: reinterpreted, never converted)
__device__ __forceinline__ float bld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
}
__device__ __forceinline__ float4 bld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 x = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
    return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
}

// Logit carry (m, E, P) of one head, wave-uniform, advanced chunk by chunk by the scan wave.
struct Carry {
    float m, E, P;
};

// Scalar scan of one chunk on one wave (lane r: token t0 + r, valid for r < nval), joined with the
// carry; writes the chunk's coefficients into parity buffer b and advances the carry. Sums of s and
// the running maximum are DPP prefix scans; the sums of e^{s} take a causal fixed reference (the
// carried maximum, or the chunk's first logit at the start of the sequence), one exponential per
// token; a lane whose running maximum exceeds the reference by more than 60 takes the exact
// (max, sum) scan instead, formed only when some lane needs it. Every lane's result depends on its
// own prefix only, so outputs never depend on later tokens, not even in rounding.
template <int C, typename Smem>
__device__ __forceinline__ void chunk_scan(Smem &sm, int b, int r, int nval, int tpos0, float s_in,
                                           float g1_in, float gh_in, float g0_in, bool has_g0, Carry &cy) {
    const bool valid = r < nval;
    const float sr = valid ? s_in : 0.f;
    const float ps = wave_scan_add(sr);
    const float mloc = wave_scan_max(valid ? sr : kNegInf);
    const float M = fmaxf(cy.m, mloc);                      // m_t
    const float ref = (cy.m == kNegInf) ? lane_f(sr, 0) : cy.m;
    const bool fixed_ok = M - ref <= 60.f;
    const float pe = wave_scan_add(valid && fixed_ok ? expf(sr - ref) : 0.f);
    float E = (exp_diff(cy.m, ref) * cy.E + pe) * expf(ref - M);
    if (__builtin_amdgcn_ballot_w64(valid && !fixed_ok) != 0) {   // the same on every lane
        float m = valid ? sr : kNegInf, e = valid ? 1.f : 0.f;
#pragma unroll
        for (int off = 1; off < C; off <<= 1) {
            const float m2 = __shfl_up(m, off, 64);
            const float e2 = __shfl_up(e, off, 64);
            if (r >= off) {
                const float Mx = fmaxf(m, m2);
                e = e * exp_diff(m, Mx) + e2 * exp_diff(m2, Mx);
                m = Mx;
            }
        }
        if (!fixed_ok) E = cy.E * exp_diff(cy.m, M) + e * exp_diff(m, M);
    }
    const float P = cy.P + ps;
    const float m_end = lane_f(M, nval - 1), E_end = lane_f(E, nval - 1), P_end = lane_f(P, nval - 1);
    if (r < C) {
        float a_loc = 0.f, a_in = 0.f, mr = 0.f, br = 0.f, gr = 0.f, es = 0.f;
        if (valid) {
            const float tt = static_cast<float>(tpos0 + r + 1);
            const float s1 = sigmoidf(g1_in), sh = sigmoidf(gh_in), s0 = has_g0 ? sigmoidf(g0_in) : 0.f;
            const float a = sh / E;
            const float d1 = s1 - sh;
            a_loc = a;
            a_in = a * exp_diff(cy.m, M);
            mr = M;
            br = d1 / tt;
            gr = -d1 * (P / tt) / tt + (s0 - sh) / tt;   // the zero-order term adds sigma0_t / t
            es = expf(sr - m_end);
        }
        sm.a_loc[b][r] = a_loc;
        sm.a_in[b][r] = a_in;
        sm.mrow[b][r] = mr;
        sm.brow[b][r] = br;
        sm.grow[b][r] = gr;
        sm.est[b][r] = es;
        sm.s[b][r] = sr;
        if (r == 0) sm.decay[b] = exp_diff(cy.m, m_end);
    }
    cy.m = m_end;
    cy.E = E_end;
    cy.P = P_end;
}

// Pass 1 needs only the running maximum: F relative to it (key weights e^{s_i - m1}, decay
// e^{m0 - m1}) and G, H unweighted by the scan.
template <int C, typename Smem>
__device__ __forceinline__ void chunk_scan_max(Smem &sm, int b, int r, int nval, float s_in, Carry &cy) {
    const bool valid = r < nval;
    const float sr = valid ? s_in : 0.f;
    const float m_end = fmaxf(cy.m, lane_f(wave_scan_max(valid ? sr : kNegInf), nval - 1));
    if (r < C) {
        sm.est[b][r] = valid ? expf(sr - m_end) : 0.f;
        sm.s[b][r] = sr;
        if (r == 0) sm.decay[b] = exp_diff(cy.m, m_end);
    }
    cy.m = m_end;
}

// Query tile of the j-th non-zero A^T tile in the order (qt, kt) = (0,0), (1,0), (1,1), (2,0), ...
__device__ __forceinline__ int tile_q(int j) { return j >= 6 ? 3 : j >= 3 ? 2 : j >= 1 ? 1 : 0; }

// Token tile tt of a chunk is finished by row half keep_half(tt) when RS = 2 (tiles {0, 3} and {1, 2}
// of a 64-token chunk: the same number of W V products per half).
__host__ __device__ constexpr int keep_half(int tt) { return (tt + (tt >> 1)) & 1; }

// RS waves share a column tile, each holding 1/RS of the state rows (RS = 2: two waves per SIMD, so
// that one wave's vector, LDS and barrier latency can overlap the other's matrix-core chains); the
// output products of the row halves are summed through LDS.
template <int D, int RS, int C, bool ROPE, bool PASS1>
__global__ __launch_bounds__(64 * (D / 16) * RS) void causal_f32_kernel(Problem p, ValuWork w, int nls) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    typedef F32Smem<D, C, RS> Smem;
    Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
    constexpr int NT = Smem::NT;            // token tiles per chunk
    constexpr int NAT = NT * (NT + 1) / 2;  // non-zero tiles of A^T
    constexpr int NW = D / 16;              // column tiles (and 16-row tiles of the states)
    constexpr int NRT = NW / RS;            // row tiles per wave
    constexpr int NWV = NW * RS;            // waves
    constexpr int SL = (NAT + NWV - 1) / NWV;   // A^T tiles per wave
    constexpr int NTH = 64 * NWV;
    constexpr int TPR = NTH / C;            // threads per token row when staging q, k
    constexpr int EPT = D / TPR;            // features per thread
    static_assert((RS == 1 || RS == 2) && NWV >= 4 && EPT % 4 == 0 && EPT <= 16 && TPR >= 2 && TPR <= 32,
                  "work split");
    static_assert(C == 32 || C == 64, "chunk size");
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), l16 = lane & 15, g4 = lane >> 4;
    const int ct = wv % NW, hh = wv / NW;   // column tile; row half (token tile kept, RS = 2)
    const int rt0 = hh * NRT;               // first row tile of this wave
    const bool scan_wave = wv == NWV - 1;

    const int nsg = PASS1 ? w.nseg - 1 : w.nseg;
    const int seg = blockIdx.x % nsg, bh = blockIdx.x / nsg;
    const int N = p.N;
    const int seg_len = w.seg_chunks * kValuChunk;   // tokens per segment (whole 64-token blocks)
    const int t_beg = min(N, seg * seg_len), t_end = min(N, (seg + 1) * seg_len);
    const int nch = (t_end - t_beg + C - 1) / C;
    // the main pass folds its last chunk only when the recurrent state is written
    const bool fold_last = PASS1 || (p.st.F != nullptr && seg == w.nseg - 1);
    const size_t row0 = static_cast<size_t>(bh) * N;
    // per-head buffers (the host keeps N d 4 bytes below 2^31); rows past N read as zero
    const uint32_t nrow_bytes = static_cast<uint32_t>(N) * D * 4, ntok_bytes = static_cast<uint32_t>(N) * 4;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const float *>(p.q) + row0 * D, nrow_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const float *>(p.k) + row0 * D, nrow_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const float *>(p.v) + row0 * D, nrow_bytes);
    const __amdgpu_buffer_rsrc_t rg1 = make_rsrc(static_cast<const float *>(p.g1) + row0, ntok_bytes);
    const __amdgpu_buffer_rsrc_t rgh = make_rsrc(static_cast<const float *>(p.gh) + row0, ntok_bytes);
    const bool has_g0 = p.g0 != nullptr;
    const __amdgpu_buffer_rsrc_t rg0 = make_rsrc(has_g0 ? static_cast<const float *>(p.g0) + row0 : nullptr,
                                                 has_g0 ? ntok_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.s + row0, ntok_bytes);
    float *o = static_cast<float *>(p.o) + row0 * D;
    // a continued sequence starts from the given state: its tokens are positions tin + 1 ...
    const bool cont = p.sin.F != nullptr;
    const int tin = cont ? p.sin.t[bh] : 0;

    // ---- staging of q^, k^ rows: thread (row lr, part lp) normalises and rotates EPT features
    const int lr = tid / TPR, lp = tid % TPR, c0 = lp * EPT;
    double rope_rev[ROPE ? EPT / 2 : 1];
    if (ROPE) {
#pragma unroll
        for (int jj = 0; jj < EPT / 2; ++jj) rope_rev[jj] = rope_rev_per_pos(c0 / 2 + jj, D, p.rope_base);
    }
    float nq[EPT], nk[EPT];
    auto load_rows = [&](const int t0) __attribute__((always_inline)) {
        const uint32_t off = static_cast<uint32_t>((t0 + lr) * D + c0) * 4;
#pragma unroll
        for (int c = 0; c < EPT; c += 4) {
            const float4 kk = bld4(rk, off + 4 * c);
            nk[c] = kk.x; nk[c + 1] = kk.y; nk[c + 2] = kk.z; nk[c + 3] = kk.w;
            if (!PASS1) {
                const float4 qq = bld4(rq, off + 4 * c);
                nq[c] = qq.x; nq[c + 1] = qq.y; nq[c + 2] = qq.z; nq[c + 3] = qq.w;
            }
        }
    };
    auto stage_rows = [&](const int bb, const int t0, const int nval) __attribute__((always_inline)) {
        const bool valid = lr < nval;
        float xq[EPT], xk[EPT];
        float ssq = 0.f, ssk = 0.f;
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            xk[c] = valid ? nk[c] : 0.f;
            ssk += xk[c] * xk[c];
            if (!PASS1) {
                xq[c] = valid ? nq[c] : 0.f;
                ssq += xq[c] * xq[c];
            }
        }
        ssk = group_sum<TPR>(ssk);
        const float ik = 1.f / fmaxf(sqrtf(ssk), 1e-12f);
        float iq = 0.f;
        if (!PASS1) {
            ssq = group_sum<TPR>(ssq);
            iq = 1.f / fmaxf(sqrtf(ssq), 1e-12f);
        }
#pragma unroll
        for (int c = 0; c < EPT; ++c) {
            xk[c] *= ik;
            if (!PASS1) xq[c] *= iq;
        }
        if (ROPE) {
            const int tok = tin + t0 + lr;      // 0-based position in the sequence
#pragma unroll
            for (int jj = 0; jj < EPT / 2; ++jj) {
                float cs, sn;
                rope_cos_sin(rope_rev[jj], tok, cs, sn);
                const float k0 = xk[2 * jj], k1 = xk[2 * jj + 1];
                xk[2 * jj] = k0 * cs - k1 * sn;
                xk[2 * jj + 1] = k0 * sn + k1 * cs;
                if (!PASS1) {
                    const float q0 = xq[2 * jj], q1 = xq[2 * jj + 1];
                    xq[2 * jj] = q0 * cs - q1 * sn;
                    xq[2 * jj + 1] = q0 * sn + q1 * cs;
                }
            }
        }
#pragma unroll
        for (int c = 0; c < EPT; c += 4) {
            *reinterpret_cast<float4 *>(&sm.kh[bb][lr][c0 + c]) = make_float4(xk[c], xk[c + 1], xk[c + 2], xk[c + 3]);
            if (!PASS1)
                *reinterpret_cast<float4 *>(&sm.qh[bb][lr][c0 + c]) = make_float4(xq[c], xq[c + 1], xq[c + 2], xq[c + 3]);
        }
    };
    // v operands of the wave's column tile: lane (l, g) takes keys 16 kt + 4 g + i of column 16 ct + l
    float vc[NT][4], vn[NT][4];
    auto load_v = [&](float(&dst)[NT][4], const int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
            const uint32_t off = static_cast<uint32_t>((t0 + 16 * kt + 4 * g4) * D + 16 * ct + l16) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[kt][i] = bld(rv, off + i * D * 4);
        }
    };

    // the first chunk's rows are read before anything else
    load_rows(t_beg);
    load_v(vc, t_beg);

    // scan inputs of one chunk on the scan wave (lane r: token t0 + r)
    float ns = 0.f, ng1 = 0.f, ngh = 0.f, ng0 = 0.f;
    auto load_scan = [&](const int t0) __attribute__((always_inline)) {
        const uint32_t off = static_cast<uint32_t>(t0 + lane) * 4;
        ns = bld(rs, off);
        if (!PASS1) {
            ng1 = bld(rg1, off);
            ngh = bld(rgh, off);
            if (has_g0) ng0 = bld(rg0, off);
        }
    };
    if (scan_wave) load_scan(t_beg);     // in flight during the carry merge below

    // ---- logit carry at the segment start (scan wave). Main pass: the given state's for the first
    // segment, else the one the combine kernel formed (the given state merged with the aggregates
    // of the 64-token blocks before the segment). Pass 1 needs only the running maximum, the
    // maximum of the given state's and of the blocks' maxima.
    Carry cy{kNegInf, 0.f, 0.f};
    if (scan_wave) {
        if (PASS1) {
            float m = (lane == 0 && cont) ? p.sin.m[bh] : kNegInf;
            const float4 *ag = w.agg + static_cast<size_t>(bh) * ((N + 63) / 64);
            for (int j = lane; j < t_beg / 64; j += 64) m = fmaxf(m, ag[j].x);
            cy.m = lane_f(wave_scan_max(m), 63);
        } else if (seg > 0) {
            const float4 c4 = w.segc[static_cast<size_t>(bh) * w.nseg + seg];
            cy = Carry{c4.x, c4.y, c4.z};
        } else if (cont) {
            cy = Carry{p.sin.m[bh], p.sin.E[bh], p.sin.P[bh]};
        }
    }

    // ---- start state in registers: the given one (first segment of the main pass), the combined
    // start state (later segments of the main pass) or zero (pass 1)
    f32x4 sF[NRT], sG[NRT], sH[NRT];
    {
        const float *S0F = nullptr, *S0G = nullptr, *S0H = nullptr;
        size_t base = static_cast<size_t>(bh) * D * D;
        if (!PASS1 && seg > 0) {
            const float *st = w.segst + (static_cast<size_t>(bh) * (w.nseg - 1) + seg - 1) * 3 * D * D;
            S0F = st;
            S0G = st + D * D;
            S0H = st + 2 * D * D;
            base = 0;
        } else if (!PASS1 && cont) {
            S0F = p.sin.F;
            S0G = p.sin.G;
            S0H = p.sin.Hs;
        }
        // one uniform branch: the loads inside issue back to back (a select per element compiles
        // to a branch and a wait per load)
        if (S0F != nullptr) {
#pragma unroll
            for (int rr = 0; rr < NRT; ++rr) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rt = rt0 + rr;
                    const size_t idx = base + static_cast<size_t>(16 * rt + 4 * g4 + i) * D + 16 * ct + l16;
                    sF[rr][i] = S0F[idx];
                    sG[rr][i] = S0G[idx];
                    sH[rr][i] = S0H[idx];
                }
            }
        } else {
#pragma unroll
            for (int rr = 0; rr < NRT; ++rr) sF[rr] = sG[rr] = sH[rr] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    if (nch > 0) {
        if (scan_wave) {
            if (PASS1) chunk_scan_max<C>(sm, 0, lane, min(C, t_end - t_beg), ns, cy);
            else chunk_scan<C>(sm, 0, lane, min(C, t_end - t_beg), tin + t_beg, ns, ng1, ngh, ng0, has_g0, cy);
            if (nch > 1) load_scan(t_beg + C);
        }
        stage_rows(0, t_beg, min(C, t_end - t_beg));
        load_rows(t_beg + C);
        load_v(vn, t_beg + C);
    }

    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const int t0 = t_beg + c * C, nval = min(C, t_end - t0);
        lds_barrier();      // q^, k^ and the coefficients of this chunk visible; W free

        // ---- A^T = K Q^T tiles (key tile kt <= query tile qt) and the weights W: tile j on wave
        // j mod NWV, the SL tiles of a wave unrolled with their own accumulators so that their
        // matrix-core chains interleave (a wave with fewer tiles repeats its last one and does not
        // store it; a wave with none skips); then the scan of the next chunk on the last wave
        if (!PASS1 && wv < NAT) {
            f32x4 acc[SL];
            int jt[SL];
#pragma unroll
            for (int k = 0; k < SL; ++k) {
                jt[k] = min(wv + k * NWV, NAT - 1);
                acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int sft = 0; sft < NW; ++sft) {
#pragma unroll
                for (int k = 0; k < SL; ++k) {
                    const int qt = tile_q(jt[k]), kt = jt[k] - qt * (qt + 1) / 2;
                    const float4 kv = ld4(&sm.kh[b][16 * kt + l16][16 * sft + 4 * g4]);
                    const float4 qv = ld4(&sm.qh[b][16 * qt + l16][16 * sft + 4 * g4]);
                    acc[k] = mfma4(kv.x, qv.x, acc[k]);
                    acc[k] = mfma4(kv.y, qv.y, acc[k]);
                    acc[k] = mfma4(kv.z, qv.z, acc[k]);
                    acc[k] = mfma4(kv.w, qv.w, acc[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < SL; ++k) {
                // lane (l, g) holds keys 16 kt + 4 g + [0, 4) of query 16 qt + l
                const int qt = tile_q(jt[k]), kt = jt[k] - qt * (qt + 1) / 2;
                const int t = 16 * qt + l16;
                const float at = sm.a_loc[b][t], mt = sm.mrow[b][t], bt = sm.brow[b][t], gt = sm.grow[b][t];
                const float4 s4 = ld4(&sm.s[b][16 * kt + 4 * g4]);
                const float si[4] = {s4.x, s4.y, s4.z, s4.w};
                float wo[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int i = 16 * kt + 4 * g4 + jj;
                    wo[jj] = (i <= t && t < nval) ? acc[k][jj] * (at * expf(si[jj] - mt) + bt * si[jj] + gt) : 0.f;
                }
                if (wv + k * NWV < NAT)
                    *reinterpret_cast<float4 *>(&sm.W[t][16 * kt + 4 * g4]) = make_float4(wo[0], wo[1], wo[2], wo[3]);
            }
        }
        if (scan_wave && c + 1 < nch) {
            const int t1 = t0 + C;
            if (PASS1) chunk_scan_max<C>(sm, b ^ 1, lane, min(C, t_end - t1), ns, cy);
            else chunk_scan<C>(sm, b ^ 1, lane, min(C, t_end - t1), tin + t1, ns, ng1, ngh, ng0, has_g0, cy);
            if (c + 2 < nch) load_scan(t1 + C);
        }

        // ---- carried-state products o^T += S^T Q^T over this wave's state rows, one token tile at a
        // time: A = the state registers, B = q^ with the contraction index in the states' row
        // order. Lane (l, g) of tile tt then holds token 16 tt + l, columns 16 ct + 4 g + [0, 4).
        f32x4 oo[NT];
        if (!PASS1) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 oF = {0.f, 0.f, 0.f, 0.f}, oG = oF, oH = oF;
#pragma unroll
                for (int rr = 0; rr < NRT; ++rr) {
                    const float4 qv4 = ld4(&sm.qh[b][16 * tt + l16][16 * (rt0 + rr) + 4 * g4]);
                    const float qv[4] = {qv4.x, qv4.y, qv4.z, qv4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        oF = mfma4(sF[rr][i], qv[i], oF);
                        oG = mfma4(sG[rr][i], qv[i], oG);
                        oH = mfma4(sH[rr][i], qv[i], oH);
                    }
                }
                const int t = 16 * tt + l16;
                const float ca = sm.a_in[b][t], cb = sm.brow[b][t], cg = sm.grow[b][t];
#pragma unroll
                for (int i = 0; i < 4; ++i) oo[tt][i] = ca * oF[i] + cb * oG[i] + cg * oH[i];
            }
            // the partials of the token tiles the other row half keeps go to it
            if constexpr (RS == 2) {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    if (keep_half(tt) != hh) sm.xch[ct][tt][lane] = make_float4(oo[tt][0], oo[tt][1], oo[tt][2], oo[tt][3]);
            }
        }

        // ---- fold the chunk's keys into the states: A = k^T (rows: features 16 rt + l), B = the
        // weighted v of the tile (keys 16 kt + 4 g + i); absent keys have zero k^ rows
        if (fold_last || c + 1 < nch) {
            const float dec = sm.decay[b];
#pragma unroll
            for (int rr = 0; rr < NRT; ++rr)
#pragma unroll
                for (int i = 0; i < 4; ++i) sF[rr][i] *= dec;
#pragma unroll
            for (int kt = 0; kt < NT; ++kt) {
                const float4 e4 = ld4(&sm.est[b][16 * kt + 4 * g4]);
                const float4 s4 = ld4(&sm.s[b][16 * kt + 4 * g4]);
                const float ev[4] = {e4.x, e4.y, e4.z, e4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float vv = vc[kt][i], be = ev[i] * vv, bs = sv[i] * vv;
#pragma unroll
                    for (int rr = 0; rr < NRT; ++rr) {
                        const float a = sm.kh[b][16 * kt + 4 * g4 + i][16 * (rt0 + rr) + l16];
                        sF[rr] = mfma4(a, be, sF[rr]);
                        sG[rr] = mfma4(a, bs, sG[rr]);
                        sH[rr] = mfma4(a, vv, sH[rr]);
                    }
                }
            }
        }

        // ---- stage the next chunk's rows (read one chunk ahead; its buffer is not read in this
        // chunk) and read the one after. Done on every chunk, without a branch, in the block of the
        // fold so that this vector work can fill the gaps of its matrix-core chain: after the last
        // chunk it stages zero rows into a buffer no longer read, and the reads past the segment
        // are in bounds or read zero past N.
        stage_rows(b ^ 1, t0 + C, min(C, t_end - t0 - C));
        load_rows(t0 + 2 * C);

        // (the fold comes before the wait for W: it takes up the time the waves forming A^T and
        // W take longer than the scan wave, or the other way round)
        if (!PASS1) {
            lds_barrier();      // W visible

            // ---- intra-chunk term W V (A = v of the tile, B = W; W[t][i] = 0 for i > t), store. With
            // RS = 2 each wave finishes the token tile of its row half, adding the other half's partial.
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                if (RS == 2 && keep_half(tt) != hh) continue;
                if constexpr (RS == 2) {
                    const float4 x = sm.xch[ct][tt][lane];
                    oo[tt][0] += x.x;
                    oo[tt][1] += x.y;
                    oo[tt][2] += x.z;
                    oo[tt][3] += x.w;
                }
#pragma unroll
                for (int kt = 0; kt <= tt; ++kt) {
                    const float4 w4 = ld4(&sm.W[16 * tt + l16][16 * kt + 4 * g4]);
                    oo[tt] = mfma4(vc[kt][0], w4.x, oo[tt]);
                    oo[tt] = mfma4(vc[kt][1], w4.y, oo[tt]);
                    oo[tt] = mfma4(vc[kt][2], w4.z, oo[tt]);
                    oo[tt] = mfma4(vc[kt][3], w4.w, oo[tt]);
                }
                const int t = 16 * tt + l16;
                if (t < nval)
                    *reinterpret_cast<float4 *>(o + static_cast<size_t>(t0 + t) * D + 16 * ct + 4 * g4) =
                        make_float4(oo[tt][0], oo[tt][1], oo[tt][2], oo[tt][3]);
            }
        }

        // ---- the v operands of the next chunk, and read the one after
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) vc[kt][i] = vn[kt][i];
        load_v(vn, t0 + 2 * C);
    }

    if (PASS1) {
        // segment-local sums (F relative to the logit maximum at the segment end) for the combine
        float *dst = w.segst + (static_cast<size_t>(bh) * (w.nseg - 1) + seg) * 3 * D * D;
#pragma unroll
        for (int rr = 0; rr < NRT; ++rr)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t idx = static_cast<size_t>(16 * (rt0 + rr) + 4 * g4 + i) * D + 16 * ct + l16;
                dst[idx] = sF[rr][i];
                dst[D * D + idx] = sG[rr][i];
                dst[2 * D * D + idx] = sH[rr][i];
            }
        if (scan_wave && lane == 0) w.segm[static_cast<size_t>(bh) * w.nseg + seg] = cy.m;
        return;
    }

    // ---- final state
    if (p.st.F != nullptr && seg == w.nseg - 1) {
        const size_t mat0 = static_cast<size_t>(bh) * D * D;
#pragma unroll
        for (int rr = 0; rr < NRT; ++rr)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t idx = mat0 + static_cast<size_t>(16 * (rt0 + rr) + 4 * g4 + i) * D + 16 * ct + l16;
                p.st.F[idx] = sF[rr][i];
                p.st.G[idx] = sG[rr][i];
                p.st.Hs[idx] = sH[rr][i];
            }
        if (tid < D) {
            float su = cont ? p.sin.Su[static_cast<size_t>(bh) * D + tid] : 0.f;
            for (int sg = 0; sg < nls; ++sg) su += w.useg[(static_cast<size_t>(bh) * nls + sg) * D + tid];
            p.st.Su[static_cast<size_t>(bh) * D + tid] = su;
        }
        if (scan_wave && lane == 0) {
            p.st.m[bh] = cy.m;
            p.st.E[bh] = cy.E;
            p.st.P[bh] = cy.P;
            p.st.t[bh] = tin + N;
        }
    }
}

template <int D, int RS, int C, bool ROPE>
hipError_t launch_v(const Problem &p, const ValuWork &w, int nls, hipStream_t stream) {
    constexpr int NTH = 64 * (D / 16) * RS;
    const size_t smem = sizeof(F32Smem<D, C, RS>);
    const void *fm = reinterpret_cast<const void *>(&causal_f32_kernel<D, RS, C, ROPE, false>);
    const void *f1 = reinterpret_cast<const void *>(&causal_f32_kernel<D, RS, C, ROPE, true>);
    hipError_t err = hipFuncSetAttribute(fm, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (err != hipSuccess) return err;
    err = hipFuncSetAttribute(f1, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (err != hipSuccess) return err;
    const int bhs = p.B * p.H;
    if (w.nseg > 1) {
        hipLaunchKernelGGL((causal_f32_kernel<D, RS, C, ROPE, true>), dim3(bhs * (w.nseg - 1)), dim3(NTH), smem,
                           stream, p, w, nls);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if ((err = launch_valu_combine(p, w, stream)) != hipSuccess) return err;
    }
    hipLaunchKernelGGL((causal_f32_kernel<D, RS, C, ROPE, false>), dim3(bhs * w.nseg), dim3(NTH), smem, stream, p,
                       w, nls);
    return hipGetLastError();
}

// One wave per column tile (RS = 1); 64-token chunks for d = 64, 32-token chunks for d = 128 (its
// 64-token variant needs more than the 256 registers of two waves per SIMD).
template <int D, bool ROPE>
hipError_t launch_d(const Problem &p, const ValuWork &w, int nls, hipStream_t stream) {
    constexpr int RS = 1, C = D == 64 ? 64 : 32;
    return launch_v<D, RS, C, ROPE>(p, w, nls, stream);
}

}  // namespace

hipError_t launch_causal_f32(const Problem &p, const ValuWork &w, hipStream_t stream) {
    const int nls = (p.N + kLogitSeg - 1) / kLogitSeg;
    switch (p.d) {
        case 64: return p.rope ? launch_d<64, true>(p, w, nls, stream) : launch_d<64, false>(p, w, nls, stream);
        case 128: return p.rope ? launch_d<128, true>(p, w, nls, stream) : launch_d<128, false>(p, w, nls, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zeros
