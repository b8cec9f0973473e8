/*
 * q4k.h -- C ABI of the MI355X (gfx950) Q4_K decode library (libq4k.so).
 *
 * The library computes the block-quantised matrix-vector products of
 * transformer decode on Q4_K weights: a plain matvec, the fused QKV
 * projection, the fused gate+up -> gated activation -> down FFN, the
 * vocabulary-sized lm_head with top-k, and a small-batch prefill matmul.
 *
 * Sources (the pages):
 *  - infer-compute README, "Shaders" table, rows "Q4_K/Q6_K" (q4k_matvec,
 *    q4k_qkv_proj) and "Q4_K fused FFN" (gate+up fused with a shared input,
 *    GELU-tanh / SiLU gated down projection); "Quick Start" (q4k_matvec takes
 *    the quantised bytes, the activation, rows and hidden size; prefill for
 *    seq > 1); "Key Optimizations" table (pre-allocated buffers, fused
 *    gate+up); "Design Principles" item 8 (Q4_K matches the GGUF format).
 *  - Performance -- infer-inference, "Activation Function Support" table
 *    (gated GELU-tanh, gated SiLU); "Honest Path Breakdown" and "Real vindex"
 *    table (lm_head on the GPU, top predictions).
 *  - infer-inference README, Overview example (top-5 predictions).
 *
 * Q4_K weight layout (GGUF super-block, 144 bytes per 256 weights):
 *   bytes 0-1  d     IEEE binary16, little-endian
 *   bytes 2-3  dmin  IEEE binary16, little-endian
 *   bytes 4-15 eight 6-bit scales sc[s] and eight 6-bit mins m[s]
 *              (s < 4: low 6 bits of bytes 4+s and 8+s; s >= 4: nibbles of
 *              byte 12+s-4 plus the top 2 bits of bytes 4+s-4 / 8+s-4)
 *   bytes 16-143 quants: byte 16+32g+r holds element 64g+r (low nibble) and
 *              element 64g+32+r (high nibble)
 *   weight e = d * sc[e/32] * q[e] - dmin * m[e/32]
 * A rows x cols matrix is rows * (cols/256) consecutive blocks, row-major; the
 * row stride is cols/256*144 bytes. cols must be a positive multiple of 256.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or keeps device memory; intermediates go in the
 *    caller's workspace `ws` (size from the matching *_workspace_bytes call).
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    on it and the call returns without synchronising; results are valid once
 *    the stream has reached that point.
 *  - Arguments are checked before anything is enqueued. On an argument error
 *    the call returns a negative q4k_status, enqueues nothing and leaves every
 *    output untouched. rows == 0 (or seq == 0) is a successful no-op.
 *  - Checks: null pointers (for non-empty tensors); cols not a positive
 *    multiple of 256 or above Q4K_COLS_MAX; negative sizes; W, x, X and
 *    workspaces not 16-byte aligned; an output range overlapping an input
 *    range or another output; unknown activation; workspace too small.
 *  - A failed kernel launch returns Q4K_ERR_HIP; q4k_last_hip_error() then
 *    returns the HIP error string (thread-local).
 *  - Calls hold no global state (apart from a per-device cache of the compute
 *    unit count) and are re-entrant; calls on one stream execute in order.
 *  - Results are deterministic: no atomics, one writer per output element.
 *
 * Activation precision (what the arithmetic of each call is):
 *  - f32 multiply-adds on the f32 activations: q4k_qkv, q6k_matvec, the down
 *    projection of q4k_ffn / q4k_rmsnorm_ffn / q4k_ffn_prefill (seq < 64), and
 *    q4k_matvec / q4k_rmsnorm_matvec / q4k_matmul (seq < 64) when a launch has
 *    few rows per compute unit.
 *  - Block floating point: the gate+up stage (q4k_gate_up, q4k_ffn,
 *    q4k_rmsnorm_ffn, q4k_ffn_prefill with seq < 64), q4k_lmhead_topk(_probs),
 *    and q4k_matvec / q4k_rmsnorm_matvec / q4k_matmul (seq < 64) with many rows
 *    per compute unit. Each 32-activation sub-block is held as 24-bit integers
 *    times a power of two when its largest magnitude is at most 6 times its
 *    mean magnitude; every activation is then within 2^-22 of the sub-block's
 *    largest magnitude (below 1.5e-6 of its mean magnitude), and the products
 *    with the 4-bit quants are exact integer dot products. Where any sub-block
 *    a wave covers is beyond that spread (an outlier activation), that wave
 *    computes with f32 multiply-adds instead, so no activation is rounded at
 *    an outlier's scale.
 *  - bf16 operands with fp32 accumulation: q4k_matmul and q4k_ffn_prefill with
 *    seq >= 64 (the matrix cores).
 *  Accumulation is f32 everywhere. The weight fields enter exactly: d, dmin
 *  (binary16), the 6-bit scales and mins and the 4-bit quants are all exact in
 *  f32, and each sub-block contributes d*sc*sum(q x) - dmin*m*sum(x).
 */
#ifndef Q4K_H
#define Q4K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum q4k_status {
    Q4K_OK = 0,
    Q4K_ERR_NULL = -1,      /* a required pointer is NULL */
    Q4K_ERR_SHAPE = -2,     /* bad rows / cols / seq / split sizes */
    Q4K_ERR_ALIGN = -3,     /* W, x, X or a workspace not 16-byte aligned */
    Q4K_ERR_K = -4,         /* top-k count outside 1..min(rows, Q4K_TOPK_MAX) */
    Q4K_ERR_ACT = -5,       /* unknown activation */
    Q4K_ERR_WORKSPACE = -6, /* workspace NULL or smaller than required */
    Q4K_ERR_ALIAS = -7,     /* an output overlaps an input or another output */
    Q4K_ERR_HIP = -8,       /* a HIP runtime/launch error */
    Q4K_ERR_EPS = -9,       /* a norm's eps negative or not finite */
    Q4K_ERR_SCRATCH = -10   /* inter above Q4K_NOALLOC_INTER_MAX (q4k_ffn_noalloc) */
};

enum q4k_act {
    Q4K_ACT_GELU_TANH = 0,  /* 0.5 z (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3))) */
    Q4K_ACT_SILU = 1        /* z / (1 + exp(-z)) */
};

#define Q4K_QK 256            /* weights per super-block */
#define Q4K_BLOCK_BYTES 144   /* bytes per Q4_K super-block */
#define Q6K_BLOCK_BYTES 210   /* bytes per Q6_K super-block */
#define Q4K_TOPK_MAX 64       /* largest k of q4k_lmhead_topk */
#define Q4K_COLS_MAX 65536    /* largest cols (reduction length) */
#define Q4K_NOALLOC_INTER_MAX 32768  /* largest inter of q4k_ffn_noalloc (128 KB of scratch) */

/* y[i] = sum_j W[i][j] * x[j], i < rows.
 * Source: infer-compute README, "Quick Start" (q4k_matvec) and "Shaders"
 * table (q4k_matvec). W: rows x cols Q4_K; x: f32[cols]; y: f32[rows]. */
int q4k_matvec(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
               void *stream);

/* y[i] = sum_j W[i][j] * x[j] for a Q6_K matrix: rows x cols, each row
 * cols/256 GGUF Q6_K blocks of 210 bytes (ql[128] low nibbles, qh[64] high
 * bit pairs, 16 signed 8-bit scales, f16 d; w = d * scale * (q - 32), one
 * scale per 16 consecutive weights). Blocks need not be aligned; W itself
 * must be 16-byte aligned. x: f32[cols]; y: f32[rows]. f32 arithmetic.
 * Source: infer-compute README, "Shaders" table (q6k_matvec) and "Design
 * Principles" item 8 (Q6_K matches the GGUF/Ollama quantisation). */
int q6k_matvec(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
               void *stream);

/* Fused QKV projection: one pass over the concatenated rows [q; k; v] of Wqkv
 * ((q_rows + 2*kv_rows) x cols), all sharing x; rows [0, q_rows) go to q,
 * [q_rows, q_rows+kv_rows) to k, the rest to v.
 * Source: infer-compute README, "Shaders" table (q4k_qkv_proj). */
int q4k_qkv(const void *Wqkv, const float *x, float *q, float *k, float *v,
            int64_t q_rows, int64_t kv_rows, int64_t cols, void *stream);

/* First FFN stage: g = Wg x and u = Wu x computed in the same pass over x
 * (Wg, Wu: inter x hidden), h[i] = act(g[i]) * u[i], h: f32[inter].
 * Source: infer-compute README, "Shaders" table (q4k_ffn_gate_up, "fused
 * gate+up, shared input") and "Activation" row (geglu_gelu_tanh/geglu_silu). */
int q4k_gate_up(const void *Wg, const void *Wu, const float *x, float *h,
                int64_t inter, int64_t hidden, int act, void *stream);

/* Workspace of q4k_ffn: the intermediate h, f32[inter] (16-byte aligned). */
size_t q4k_ffn_workspace_bytes(int64_t hidden, int64_t inter);

/* Gated FFN for one token: h = act(Wg x) * (Wu x) (q4k_gate_up), then
 * y = Wd h (Wd: hidden x inter). x: f32[hidden]; y: f32[hidden]; h lives in
 * ws. Source: infer-compute README, "Shaders" table (q4k_ffn_gate_up
 * followed by q4k_geglu_gelu_tanh_down / q4k_geglu_silu_down). */
int q4k_ffn(const void *Wg, const void *Wu, const void *Wd, const float *x, float *y,
            int64_t hidden, int64_t inter, int act, void *ws, size_t ws_bytes, void *stream);

/* q4k_ffn for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the intermediate h
 * lives in a scratch array inside the library instead of a caller workspace,
 * so there is no workspace argument and the call allocates nothing. The
 * scratch holds Q4K_NOALLOC_INTER_MAX floats per device (128 KB, kept until
 * the process ends); a larger inter returns Q4K_ERR_SCRATCH. Every call on a
 * device shares that device's scratch: calls that overlap on one device (on
 * different streams, or from different threads) race and give wrong results;
 * calls on one stream are ordered and safe. Nothing in it must start at
 * zero. Outputs equal q4k_ffn's bit for bit (the same kernels). */
int q4k_ffn_noalloc(const void *Wg, const void *Wu, const void *Wd, const float *x, float *y,
                    int64_t hidden, int64_t inter, int act, void *stream);

/* Residual RMSNorm fused into a projection's input (the residual_norm step
 * before a layer's projections):
 *   s = h + delta   (f32 addition; delta may be NULL: s = h),
 *   x = s / sqrt(mean(s^2) + eps) * norm_w,   y = W x.
 * h, delta, norm_w: f32[cols]; h_out (may be NULL) receives s, the updated
 * residual stream, and must not overlap any other argument (in particular not
 * h: other workgroups still read h while it is written). A model whose norm
 * scales by (1 + w) passes 1 + w as norm_w. The scalar 1/sqrt(...) is applied
 * to each output row; (s * norm_w) is what the weights multiply. eps must be
 * finite and >= 0 (else Q4K_ERR_EPS); rows must be >= 1. For a fused QKV
 * projection pass Wqkv with rows = q_rows + 2*kv_rows: q, k, v are then the
 * consecutive slices of y. h, delta, norm_w, h_out: 16-byte aligned.
 * Source: infer-compute README, "Key Optimizations" table (cooperative
 * rms_norm / residual_norm) and "Shaders" table (fused residual_norm);
 * Performance -- infer-inference, "Norm comparison" table (RMSNorm). */
int q4k_rmsnorm_matvec(const void *W, const float *h, const float *delta, const float *norm_w,
                       float eps, float *h_out, float *y, int64_t rows, int64_t cols,
                       void *stream);

/* q4k_ffn with the same residual RMSNorm fused into the gate+up input
 * (hidden = the norm's length); the down projection reads h as in q4k_ffn.
 * Workspace: q4k_ffn_workspace_bytes. */
int q4k_rmsnorm_ffn(const void *Wg, const void *Wu, const void *Wd, const float *h,
                    const float *delta, const float *norm_w, float eps, float *h_out, float *y,
                    int64_t hidden, int64_t inter, int act, void *ws, size_t ws_bytes,
                    void *stream);

/* Largest vocabulary (rows) q4k_lmhead_topk and q4k_lmhead_topk_probs accept
 * for this cols (0 for an invalid cols): about 4.18 million rows at cols 2560.
 * Beyond it the calls return Q4K_ERR_SHAPE (the per-workgroup candidate lists
 * would exceed what the merge takes). */
int64_t q4k_lmhead_rows_max(int64_t cols);

/* Workspace of q4k_lmhead_topk and q4k_lmhead_topk_probs: per-workgroup
 * top-k candidates and softmax partials (0 for an invalid shape or k, or rows
 * above q4k_lmhead_rows_max(cols)). */
size_t q4k_lmhead_workspace_bytes(int64_t rows, int64_t cols, int k);

/* logits = W x over all rows (the vocabulary), then the k largest logits in
 * order of value descending, index ascending (NaN logits rank last).
 * top_idx: int32[k]; top_val: f32[k] (the logits at those rows). Requires
 * 1 <= k <= min(rows, Q4K_TOPK_MAX) (else Q4K_ERR_K) and
 * rows <= q4k_lmhead_rows_max(cols) (else Q4K_ERR_SHAPE).
 * Source: Performance -- infer-inference, "Honest Path Breakdown" (GPU
 * logits) and "Real vindex" table (lm_head); infer-inference README, Overview
 * example (top-5 predictions). */
int q4k_lmhead_topk(const void *W, const float *x, float *logits, int64_t rows, int64_t cols,
                    int k, int32_t *top_idx, float *top_val, void *ws, size_t ws_bytes,
                    void *stream);

/* q4k_lmhead_topk, plus the softmax over all rows' logits:
 * lse[0] = log sum_i exp(logits[i]) and top_prob[r] = exp(top_val[r] - lse),
 * the probability of the r-th prediction (f32[k]). Computed in f32 in the same
 * pass: each workgroup reduces (max, sum of exp(l - max)) over its rows and
 * the merge combines them. A NaN logit makes lse and every top_prob NaN.
 * top_prob and lse must not overlap each other or any other argument.
 * Source: infer-inference README, Overview example (top prediction printed
 * with its probability); Performance -- infer-inference, "Real vindex" table
 * (top prediction with its probability). */
int q4k_lmhead_topk_probs(const void *W, const float *x, float *logits, int64_t rows,
                          int64_t cols, int k, int32_t *top_idx, float *top_val, float *top_prob,
                          float *lse, void *ws, size_t ws_bytes, void *stream);

/* Workspace of q4k_matmul (bf16 copy of X for seq >= 64; 0 otherwise). */
size_t q4k_matmul_workspace_bytes(int64_t rows, int64_t cols, int64_t seq);

/* Small-batch matmul for prefill: Y[t][i] = sum_j W[i][j] X[t][j],
 * X: f32[seq][cols], Y: f32[seq][rows] (token-major). seq >= 64 runs on the
 * matrix cores with bf16 operands (weights dequantised to bf16 tiles in LDS,
 * fp32 accumulation); smaller seq runs the f32 matvec of every token in one
 * launch (the same per-row arithmetic as q4k_matvec, so each Y row equals
 * q4k_matvec of that token bit for bit).
 * Source: infer-compute README, "Quick Start" (GPU prefill for seq > 1). */
int q4k_matmul(const void *W, const float *X, float *Y, int64_t rows, int64_t cols,
               int64_t seq, void *ws, size_t ws_bytes, void *stream);

/* Workspace of q4k_ffn_prefill (seq < 64: h for every token, f32[seq][inter]). */
size_t q4k_ffn_prefill_workspace_bytes(int64_t seq, int64_t hidden, int64_t inter);

/* Gated FFN for seq tokens: H = act(X Wg^T) * (X Wu^T), Y = H Wd^T.
 * X, Y: f32[seq][hidden]. seq >= 64: bf16 matrix-core path with the gated
 * activation applied to fp32 G/U before H is rounded to bf16; smaller seq:
 * the f32 gate+up of every token in one launch, then the down projection of
 * every token in one launch (each Y row equals q4k_ffn of that token bit for
 * bit). Source: infer-compute README, "Quick Start" (prefill)
 * and "Shaders" table (Q4_K fused FFN row). */
int q4k_ffn_prefill(const void *Wg, const void *Wu, const void *Wd, const float *X, float *Y,
                    int64_t seq, int64_t hidden, int64_t inter, int act,
                    void *ws, size_t ws_bytes, void *stream);

/* Measurement helpers (not part of the decode path): the device-side
 * counterparts of the pages' bandwidth and raw-dispatch profiles
 * (infer-compute README, "Benchmarks: Profile (bottleneck analysis)").
 *
 * q4k_probe_read streams `bytes` bytes of the device buffer buf with the same
 * unconditional 128-bit buffer loads as the decode kernels: `grid` workgroups
 * of `threads` threads (a multiple of 64, at most 1024), each thread issuing
 * `depth` loads (1, 2, 4, 8 or 16) before using their data; contiguous = 0
 * strides the whole grid through the buffer (thread g reads the 16 bytes at
 * (i * grid * threads + g) * 16), contiguous != 0 gives each workgroup one
 * contiguous share. bytes: a positive multiple of 16 below 2^31; buf 16-byte
 * aligned. sink: 4 device bytes the kernel may write (it keeps the loads from
 * being optimised away) and that must not overlap buf.
 * q4k_probe_empty launches a kernel with an empty body (grid x threads) into
 * sink's stream position: the cost of one launch.
 * Errors: Q4K_ERR_SHAPE (sizes, grid, threads, depth), Q4K_ERR_NULL,
 * Q4K_ERR_ALIGN, Q4K_ERR_ALIAS, Q4K_ERR_HIP. */
int q4k_probe_read(const void *buf, int64_t bytes, int grid, int threads, int depth,
                   int contiguous, uint32_t *sink, void *stream);
int q4k_probe_empty(int grid, int threads, uint32_t *sink, void *stream);

/* Human-readable name of a q4k_status value (static string). */
const char *q4k_status_string(int status);

/* The HIP error string of the last Q4K_ERR_HIP on this thread ("" if none). */
const char *q4k_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4K_H */
