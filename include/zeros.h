/*
 * libzeros: ZeroS (zero-sum linear attention) for AMD Instinct MI355X (gfx950): the causal and
 * encoder forward passes, the recurrent decode step, the backward of the causal forward, and the
 * quadratic variant ZeroS-SM.
 *
 * The method (arXiv 2602.05230) is described on the Paper-Notes page "ZeroS: Zero-Sum Linear
 * Attention for Efficient Transformers" (section 关键设计) and on the ai.info summary of the same
 * title (section "Methodology in Plain English"). Per head, with 1-based positions t and i:
 *
 *   deviation logits      s_i  = -(u_i . ubar_i) / sqrt(d_u),
 *                         ubar_i = (e^tau mu + sum_{j<=i} u_j) / (e^tau + i)
 *   zero-sum weights      w_{t,i} = sigma1_t (s_i - P_t/t)/t
 *                                 + sigmah_t (softmax_{t,i} - 1/t - (s_i - P_t/t)/t)
 *   angular factor        cos_{t,i} = q^_t . k^_i  (L2-normalised, optionally RoPE-rotated)
 *   output                o_t = sum_{i<=t} w_{t,i} cos_{t,i} v_i
 *                             = q^_t (alpha_t F_t + beta_t G_t + gamma_t H_t)
 *
 * with E_t = sum e^{s_i}, P_t = sum s_i, F_t = sum e^{s_i} k^_i^T v_i, G_t = sum s_i k^_i^T v_i,
 * H_t = sum k^_i^T v_i (the prefix scan of 关键设计 / 线性时间前缀扫描), alpha_t = sigmah_t/E_t,
 * beta_t = (sigma1_t - sigmah_t)/t, gamma_t = -(sigma1_t - sigmah_t) P_t/t^2 - sigmah_t/t, and
 * sigma = logistic sigmoid of the gate pre-activations g1, gh.
 *
 * Optional zero-order gate (Paper-Notes 关键设计, the design motivation of the zero-order removal:
 * a first layer may keep the uniform term; ai.info "Methodology in Plain English": a gate
 * sigma0_t decides how much of it to keep): when g0 is not NULL every weight of row t gains
 * sigma0_t / t, i.e. gamma_t += sigmoid(g0_t) / t (t = N in the encoder). The weights then sum
 * to sigma0_t instead of zero. g0 = NULL leaves the term out (the pages' default).
 *
 * Conventions shared by every entry point
 *   Memory:    every pointer is DEVICE memory owned by the caller; the library allocates no
 *              memory at run time and keeps no state between calls (an error message is kept
 *              per thread, a per-device flag records that a kernel attribute was set, and the
 *              device address of the fixed scratch array of zeros_fwd_causal_noalloc is kept
 *              per device). Scratch memory comes from the caller as a workspace argument whose
 *              size a *_workspace_bytes query gives; a call that needs scratch and gets none
 *              returns ZEROS_ERR_NULL.
 *              Token tensors (q, k, v, u, g1, gh, o) may be NULL when N = 0; mu and tau never;
 *              g0 may always be NULL.
 *   Layout:    contiguous row-major, feature dimension innermost:
 *              q, k, v, o [B, H, N, d]; u [B, H, N, d_u]; g1, gh, g0 [B, H, N];
 *              mu [H, d_u] float32; tau [H] float32 (per head, shared across the batch).
 *   Types:     q, k, v, u, g1, gh, g0 and o share `dtype` (float32 or bfloat16); arithmetic is
 *              float32 (states, sums and accumulation); o is written in `dtype`.
 *   Streams:   work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *              returns without synchronising.
 *   Errors:    the return value only; nothing throws or aborts. Arguments are validated on the
 *              host before any launch; a failed launch returns ZEROS_ERR_HIP. NaN/Inf in the
 *              inputs propagate to the outputs they influence and are not checked.
 *   Alignment: q, k, v, u and o must be 16-byte aligned (ZEROS_ERR_SHAPE otherwise).
 *   Aliasing:  o must not overlap any input; a state the call writes must not overlap the other
 *              arguments or itself (ZEROS_ERR_ALIAS). Decode updates its state in place.
 *   Shapes:    d in {16, 32, 64, 128}, d_u == d, B, H >= 1, N >= 0 (N = 0 computes no output;
 *              a causal call with state_out still writes the state),
 *              B*H*N*d < 2^31 elements per tensor; anything else is ZEROS_ERR_UNSUPPORTED or
 *              ZEROS_ERR_SHAPE.
 *   Threads:   calls are thread-safe; calls that write the same buffers race.
 */
#ifndef ZEROS_H
#define ZEROS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZEROS_ABI_VERSION 4

typedef enum {
    ZEROS_OK = 0,
    ZEROS_ERR_NULL = 1,         /* a required pointer is NULL                         */
    ZEROS_ERR_SHAPE = 2,        /* non-positive or overflowing sizes, d_u != d        */
    ZEROS_ERR_DTYPE = 3,        /* dtype is not a zeros_dtype value                   */
    ZEROS_ERR_UNSUPPORTED = 4,  /* valid but not implemented (e.g. d = 96)             */
    ZEROS_ERR_HIP = 5,          /* the HIP runtime reported an error                  */
    ZEROS_ERR_ALIAS = 6         /* o overlaps an input                                 */
} zeros_status;

typedef enum { ZEROS_F32 = 0, ZEROS_BF16 = 1 } zeros_dtype;

typedef struct {
    int32_t B, H, N;      /* batch (or decode sequences), heads, tokens                 */
    int32_t d, d_u;       /* head dim of q/k/v/o, logit dim of u and mu                  */
    int32_t dtype;        /* zeros_dtype                                                  */
    int32_t rope;         /* 0: off; 1: RoPE on interleaved pairs (2j, 2j+1), applied to  */
                          /*    q^ and k^ after normalisation at 0-based position t-1     */
    float rope_base;      /* theta_j = rope_base^(-2j/d); 10000 is the usual value        */
} zeros_shape;

/*
 * Recurrent state of S sequences x H heads, all float32 except t. F is kept rescaled by the
 * running maximum of the logits: F = sum_i e^{s_i - m} k^_i^T v_i and E = sum_i e^{s_i - m};
 * G, Hs, P, Su are plain sums. Matrices are [S, H, d, d] with the k^ index as rows and the v
 * index as columns. The state at t = 0 is m = -inf and everything else zero. F, G and Hs must be
 * 16-byte aligned and the other fields 4-byte aligned (ZEROS_ERR_SHAPE otherwise).
 */
typedef struct {
    float *F, *G, *Hs;    /* [S, H, d, d]                                                 */
    float *Su;            /* [S, H, d_u]  running sum of u                                 */
    float *m, *E, *P;     /* [S, H]       running max, sum e^{s-m}, sum s                  */
    int32_t *t;           /* [S, H]       tokens consumed                                  */
} zeros_state;

/*
 * Causal forward (Paper-Notes 关键设计: zero-sum weights, radial-angular decoupling, deviation
 * logits and the linear-time prefix scan; decoder mode per 损失函数 / 训练策略).
 * Inputs as in the conventions above; writes o [B, H, N, d].
 * state_in (nullable): continue every (b, h) from this state (S = B) instead of the empty one:
 *   the N tokens are positions state_in.t + 1 ... state_in.t + N of their sequences (logit
 *   running mean, coefficients and RoPE angles included), as if the earlier tokens had been
 *   part of the call (chunked prefill). Heads may have consumed different numbers of tokens.
 *   Read only. bfloat16 d 64/128 calls stay on the matrix-core path (the state enters in its
 *   centred basis); the others, and a call with N = 0, take the float32 path. Its contents are
 *   device data and are not checked: it must be a state as this library writes it (t >= 0;
 *   m finite and E > 0 when t > 0; the empty state otherwise), else the outputs are undefined.
 * state_out (nullable): receives the state after the call's last token for every (b, h) (S = B);
 *   its buffers must not overlap the inputs, state_in, o or each other (ZEROS_ERR_ALIAS; continue
 *   in place by alternating two states).
 * workspace: device scratch of at least zeros_fwd_causal_workspace_bytes(shape) bytes,
 *   256-byte aligned, owned by the caller and used only while the call's work runs on `stream`
 *   (it holds the logits s_i, per-segment u sums, per-64-token logit aggregates, the scan's
 *   segment states when a head is split into segments, and on the bfloat16 d = 64/128 path the
 *   per-64-token-chunk scalar coefficients, 2.6 KB per chunk; 68.6 MB in all at B=2 H=16
 *   N=16384 d=128, half the bytes of q). NULL is
 *   ZEROS_ERR_NULL whenever the query returns more than 0 (it does for every N > 0); a workspace
 *   smaller than required or not 256-byte aligned is ZEROS_ERR_SHAPE.
 */
zeros_status zeros_fwd_causal(const zeros_shape *shape,
                              const void *q, const void *k, const void *v, const void *u,
                              const float *mu, const float *tau,
                              const void *g1, const void *gh, const void *g0,
                              void *o, const zeros_state *state_in, const zeros_state *state_out,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes zeros_fwd_causal needs for `shape`, with or without state_in (0 if it needs none,
 * or if shape is invalid). Depends on B, H, N, d, d_u and dtype only. */
size_t zeros_fwd_causal_workspace_bytes(const zeros_shape *shape);

/*
 * zeros_fwd_causal without a workspace and without any allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, results and validation as zeros_fwd_causal; the scratch is
 * a fixed array of ZEROS_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, held from the
 * library's load until the process ends. A call whose zeros_fwd_causal_workspace_bytes exceeds
 * that size returns ZEROS_ERR_UNSUPPORTED before any launch. Every call on one GPU uses that GPU's
 * array, so calls that overlap in time on the same GPU (on different streams, or from different
 * threads without ordering) race and give undefined results; calls ordered on one stream are
 * safe. No part of the array needs to start at zero (every region is written before it is read
 * within a call). The first call on a device resolves the array's device address
 * (hipGetSymbolAddress) and keeps it.
 */
#define ZEROS_NOALLOC_SCRATCH_BYTES (64u << 20)
zeros_status zeros_fwd_causal_noalloc(const zeros_shape *shape,
                                      const void *q, const void *k, const void *v, const void *u,
                                      const float *mu, const float *tau,
                                      const void *g1, const void *gh, const void *g0,
                                      void *o, const zeros_state *state_in, const zeros_state *state_out,
                                      void *stream);

/*
 * Encoder (non-causal) forward (Paper-Notes 损失函数 / 训练策略: both modes are supported).
 * Every query t uses the sums over all N tokens, ubar is the single prior-smoothed mean of all
 * N u's, and the coefficients use t = N with the gates of token t. Writes o [B, H, N, d].
 * workspace: device scratch of zeros_fwd_encoder_workspace_bytes(shape) bytes, 256-byte aligned,
 *   owned by the caller and used only while the call's work runs on `stream`. Only bfloat16
 *   calls with d 64/128 and N > 4096 need any (per (b, h): the logits, u sums per 256 tokens,
 *   and three float32 d x d partial states per block of 256 to 2048 tokens); for every other
 *   shape it may be NULL. NULL when scratch is needed is ZEROS_ERR_NULL; too small or not
 *   256-byte aligned is ZEROS_ERR_SHAPE.
 */
zeros_status zeros_fwd_encoder(const zeros_shape *shape,
                               const void *q, const void *k, const void *v, const void *u,
                               const float *mu, const float *tau,
                               const void *g1, const void *gh, const void *g0,
                               void *o, void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes zeros_fwd_encoder needs for `shape` (0 if it needs none, or if shape is invalid). */
size_t zeros_fwd_encoder_workspace_bytes(const zeros_shape *shape);

/*
 * One recurrent step (the O(d^2)-per-token update of 关键设计 / 线性时间前缀扫描):
 * shape->B = S sequences, shape->N must be 1. q, k, v, o [S, H, d]; u [S, H, d_u];
 * g1, gh, g0 [S, H]. Each (sequence, head) consumes one token at position state.t + 1 and its state
 * is updated in place; the state must not overlap the token tensors, mu, tau or o, and its
 * fields must not overlap each other (ZEROS_ERR_ALIAS).
 */
zeros_status zeros_decode_step(const zeros_shape *shape,
                               const void *q, const void *k, const void *v, const void *u,
                               const float *mu, const float *tau,
                               const void *g1, const void *gh, const void *g0,
                               void *o, const zeros_state *state, void *stream);

/*
 * Backward of the causal forward (training uses the module in place of attention: Paper-Notes
 * 损失函数 / 训练策略; the gradients follow the chain rule through the explicit weights of
 * 关键设计): given the upstream gradient dO [B, H, N, d] of o, writes the gradients of
 * L = sum_t dO_t . o_t with respect to every input: dq, dk, dv [B, H, N, d], du [B, H, N, d_u],
 * dg1, dgh (and dg0 when g0 is given, else it must be NULL) [B, H, N], all in `dtype`, and
 * dmu [H, d_u], dtau [H] in float32, summed over the batch (mu and tau are per head). The
 * forward is recomputed from the inputs (the empty initial state; no state_in / state_out).
 * Arithmetic is float32 throughout for both dtypes. Gradients must not overlap the inputs, dO or
 * each other (ZEROS_ERR_ALIAS); dO, dq, dk, dv, du 16-byte aligned, dmu and dtau 4-byte
 * aligned. workspace: zeros_bwd_causal_workspace_bytes(shape) bytes, 256-byte aligned, caller-
 * owned, used while the call's work runs on `stream` (float32 copies of q^, k^, v, dO, the three
 * scans' results and per-token scalars: about 7 N d + 20 N floats per (b, h)); NULL when needed is
 * ZEROS_ERR_NULL. N = 0 writes zero dmu and dtau.
 */
zeros_status zeros_bwd_causal(const zeros_shape *shape,
                              const void *q, const void *k, const void *v, const void *u,
                              const float *mu, const float *tau,
                              const void *g1, const void *gh, const void *g0, const void *dO,
                              void *dq, void *dk, void *dv, void *du, float *dmu, float *dtau,
                              void *dg1, void *dgh, void *dg0,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes zeros_bwd_causal needs for `shape` (0 for invalid sizes). */
size_t zeros_bwd_causal_workspace_bytes(const zeros_shape *shape);

/*
 * ZeroS-SM, causal (ai.info page "ZeroS: Zero-Sum Linear Attention for Efficient Transformers",
 * Methodology in Plain English: the same zero-sum reweighting applied to standard softmax
 * attention, the quadratic-time variant; the split and the gates as in the Paper-Notes page,
 * 关键设计). With l_{t,i} = q_t . k_i / sqrt(d) for i <= t (q, k rotated by RoPE at their 0-based
 * positions when shape->rope is 1), p_t = softmax over i of l_{t,i}, delta_{t,i} = l_{t,i} minus the
 * row mean:  o_t = sum_{i<=t} [sigma1_t delta_{t,i}/t + sigmah_t (p_{t,i} - 1/t - delta_{t,i}/t)
 * (+ sigma0_t/t)] v_i, sigma = sigmoid of g1, gh (g0: NULL for none). The pages give ZeroS-SM only
 * by that sentence; this reading is the plainest one (no cosine factor: the logits carry it).
 * q, k, v, o [B, H, N, d]; g1, gh, g0 [B, H, N]; bfloat16 only (ZEROS_ERR_UNSUPPORTED otherwise),
 * d = 64 or 128, float32 accumulation; shape->d_u is not used (any value >= 1). o must not overlap
 * an input; q, k, v, o 16-byte aligned. workspace: zeros_sm_fwd_causal_workspace_bytes(shape) bytes
 * (the rotated q and k with RoPE, else 0 and it may be NULL), 256-byte aligned, caller-owned, used
 * while the call's work runs on `stream`.
 */
zeros_status zeros_sm_fwd_causal(const zeros_shape *shape, const void *q, const void *k, const void *v,
                                 const void *g1, const void *gh, const void *g0, void *o,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes zeros_sm_fwd_causal needs for `shape` (0 without RoPE or for invalid sizes). */
size_t zeros_sm_fwd_causal_workspace_bytes(const zeros_shape *shape);

/* Bytes of one state for S x H heads when packed by zeros_state_from_buffer (256-B aligned
 * fields, order F, G, Hs, Su, m, E, P, t). Returns 0 for invalid sizes. */
size_t zeros_state_bytes(int32_t S, int32_t H, int32_t d, int32_t d_u);

/* Point the fields of *out into one buffer of zeros_state_bytes() bytes (no device access). */
zeros_status zeros_state_from_buffer(void *base, int32_t S, int32_t H, int32_t d, int32_t d_u,
                                     zeros_state *out);

/* Static description of a status code. */
const char *zeros_status_str(int32_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *zeros_last_error(void);

/* ZEROS_ABI_VERSION of the built library. */
int32_t zeros_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZEROS_H */
