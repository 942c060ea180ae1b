// Internal interface between the C-ABI front end (zeros_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/zeros.h"

namespace zeros {

// Everything a kernel needs, validated by the front end. Pointers are device pointers.
struct Problem {
    const void *q, *k, *v, *u;
    const float *mu, *tau;
    const void *g1, *gh;
    const void *g0;     // zero-order gate pre-activations, or NULL (term off)
    void *o;
    zeros_state st;     // all NULL when no state is read or written
    zeros_state sin;    // causal: state to continue from (all NULL: the empty state)
    int B, H, N, d, du;
    int dtype;          // zeros_dtype
    int rope;
    float rope_base;
};

// Tokens per segment of the two-pass logit computation, and per chunk of the causal scan.
constexpr int kLogitSeg = 256;
constexpr int kCausalChunk = 64;

// Per-chunk scalar scan and coefficients of the causal MFMA path (written by its coefficient
// kernel, read by both scan passes).
struct Coef {
    float qa[kCausalChunk], qm[kCausalChunk], qb[kCausalChunk], qg[kCausalChunk];   // per query t
    float qcx[kCausalChunk], qkap[kCausalChunk];
    float wx[kCausalChunk], wy[kCausalChunk], s[kCausalChunk], ek[kCausalChunk];     // per key i
    float chunk[8];          // m1, E1, P1, rX, cHX, cHY, exact-exp flag (chunk end / chunk map)
};

// Workspace of the causal MFMA path, carved from one caller- or library-provided buffer.
struct CausalWork {
    float *s;           // [B*H, N] logits
    float *useg;        // [B*H, nseg, d_u] per-segment u sums
    float4 *agg;        // [B*H, nchunk] per-chunk (max s, sum e^{s-max}, sum s, 0)
    float4 *segsc;      // [B*H, nseg] composed scalar map (Rs, Hs, Ys, 0) of each scan segment
    float *segst;       // [B*H, nseg-1, 3, d, d] segment-local sums, then segment start states
    uint16_t *sink;     // [kCausalChunk, d] bf16: output rows past N are written here and ignored
    int nseg;           // scan segments per head
    int seg_chunks;     // chunks per segment (the last one may be shorter)
    Coef *coef;         // [B*H, nchunk] scalar scan and coefficients of each chunk
};
size_t causal_work_bytes(int B, int H, int N, int du);
CausalWork causal_work_carve(void *base, int B, int H, int N, int du);

// Workspace of the float32 / small-d causal path (logits computed ahead of the scan kernel). Its
// segment plan counts in chunks of kValuChunk tokens.
constexpr int kValuChunk = 32;
struct ValuWork {
    float *s;           // [B*H, N] logits
    float *useg;        // [B*H, ceil(N/kLogitSeg), d_u] u sums per logit segment
    float4 *agg;        // [B*H, ceil(N/64)] per-64-token logit aggregates (segment start carries)
    float *segst;       // [B*H, nseg-1, 3, d, d] segment-local F, G, H, then segment start states
    float *segm;        // [B*H, nseg] running logit maximum at the end of each segment
    float4 *segc;       // [B*H, nseg] logit carry (m, E, P, 0) at the start of each segment
    int nseg;           // scan segments per head (1: a single pass)
    int seg_chunks;     // 32-token chunks per segment (even: segments start on 64-token blocks)
};
size_t causal_valu_work_bytes(int B, int H, int N, int du);
ValuWork causal_valu_work_carve(void *base, int B, int H, int N, int du);
hipError_t launch_causal_valu(const Problem &p, const ValuWork &w, hipStream_t stream);
// Pieces of the float32 path: the combine of the segment states (segmented scans), and the per-head
// scan kernels for float32 with d in {64, 128} (logits already in the workspace).
hipError_t launch_valu_combine(const Problem &p, const ValuWork &w, hipStream_t stream);
hipError_t launch_causal_f32(const Problem &p, const ValuWork &w, hipStream_t stream);

// Logits of the causal paths: s [B*H, N], the u sums per 256-token segment and the 64-token
// (max, sum e^{s - max}, sum s) aggregates.
hipError_t launch_logits(const Problem &p, float *useg, float *s_out, float4 *agg, hipStream_t stream);
// Column sums of u per 256-token segment alone [B*H, ceil(N/256), d] (d 64 or 128).
hipError_t launch_usum(const Problem &p, float *useg, hipStream_t stream);
hipError_t launch_causal_mfma(const Problem &p, const CausalWork &w, hipStream_t stream);
// Encoder: `work` is caller scratch of encoder_work_bytes(p) bytes (NULL when that is 0).
hipError_t launch_encoder(const Problem &p, void *work, hipStream_t stream);
// Matrix-core encoder for bfloat16, d in {64, 128}. Sequences of up to 256 tokens, and those below
// kEncoderTileMaxN tokens while q holds fewer than kEncoderLongElems elements, run in one launch
// (encoder_mfma.hip: one workgroup per head, or per (head, 16-column tile) with the logits in LDS).
// The others take the token-parallel pipeline of encoder_long.hip: five launches over (head, block
// of tokens), whose scratch is encoder_long_work_bytes(p) bytes. (Measured crossover: the single
// launch repeats its logits pass per column tile and has few workgroups per head, the pipeline
// costs about 20 us of launches.)
constexpr int kEncoderTileMaxN = 768;
constexpr long kEncoderLongElems = 6291456;     // 96 Ki tokens at d = 64
inline bool encoder_long_path(const Problem &p) {
    return p.N > 256 &&
           (p.N >= kEncoderTileMaxN || static_cast<long>(p.B) * p.H * p.N * p.d >= kEncoderLongElems);
}
size_t encoder_work_bytes(const Problem &p);
size_t encoder_long_work_bytes(const Problem &p);
hipError_t launch_encoder_long(const Problem &p, void *work, hipStream_t stream);
hipError_t launch_encoder_mfma(const Problem &p, hipStream_t stream);
hipError_t launch_decode(const Problem &p, hipStream_t stream);

// ZeroS-SM, the zero-sum reweighting of standard causal softmax attention (sm_causal.hip):
// bfloat16, d = 64 or 128; with RoPE, `work` holds the rotated q and k (sm_work_bytes).
size_t sm_work_bytes(const Problem &p);
hipError_t launch_sm_causal(const Problem &p, void *work, hipStream_t stream);

// Backward of the causal forward (backward.hip). Gradient outputs in the storage dtype except
// dmu [H, d_u] and dtau [H] (float32, summed over the batch).
struct BwdGrads {
    const void *dO;
    void *dq, *dk, *dv, *du;
    float *dmu, *dtau;
    void *dg1, *dgh, *dg0;     // dg0 NULL when the zero-order gate is off
};
// Float32 scratch of the backward, carved from the caller's workspace.
struct BwdWork {
    float *s, *m, *E, *P, *al, *be, *ga, *s1, *sh, *s0, *ds;   // [B*H, N] per token
    float4 *agg;                                               // [B*H, ceil(N/64)] (logits kernel)
    float *qh, *kh, *vf, *dOf, *dqh, *dkh, *dvf;               // [B*H, N, d]
    float *dotsA, *dotsB;                                      // [d/16, 3 or 2, B*H, N]
    float *useg, *dseg, *dmu_p, *dtau_p;                       // [B*H, ceil(N/256), d_u]
};
size_t causal_bwd_work_bytes(int B, int H, int N, int d);
BwdWork causal_bwd_work_carve(void *base, int B, int H, int N, int d);
hipError_t launch_causal_bwd(const Problem &p, const BwdGrads &g, const BwdWork &w, hipStream_t stream);

}  // namespace zeros
