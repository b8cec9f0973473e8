// C ABI of libq4k.so: argument checking, workspace carving and dispatch.
// Every check runs before anything is enqueued, so a failing call leaves the
// stream and all outputs untouched. Semantics of each call: include/q4k.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "q4k.h"
#include "q4k_internal.h"

#define Q4K_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_hip_error[256] = "";

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return Q4K_OK;
    snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e),
             hipGetErrorString(e));
    return Q4K_ERR_HIP;
}

// Status of a call's launches. Built with Q4K_DEBUG_SYNC, the call also waits
// for its stream and reports a kernel that failed while running (a debugging
// aid: such a build cannot be captured into a graph).
int finish(hipError_t e, hipStream_t s)
{
#ifdef Q4K_DEBUG_SYNC
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
#else
    (void)s;
#endif
    return hip_status(e);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Half-open byte range of a tensor; empty ranges overlap nothing.
struct Span {
    uintptr_t lo, hi;
};
Span span(const void *p, int64_t bytes) { return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }
bool overlap(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool cols_ok(int64_t cols) { return cols > 0 && cols % Q4K_QK == 0 && cols <= Q4K_COLS_MAX; }
bool rows_ok(int64_t rows) { return rows >= 0 && rows <= INT32_MAX; }
int64_t wbytes(int64_t rows, int64_t cols) { return rows * (cols / Q4K_QK) * Q4K_BLOCK_BYTES; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int64_t kMfmaMinSeq = 64;  // seq at which prefill switches to the matrix cores
constexpr int64_t kSeqMax = 64 * 65535;  // 64-token groups on one grid dimension

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

Q4K_EXPORT const char *q4k_status_string(int status)
{
    switch (status) {
        case Q4K_OK: return "Q4K_OK";
        case Q4K_ERR_NULL: return "Q4K_ERR_NULL: a required pointer is NULL";
        case Q4K_ERR_SHAPE: return "Q4K_ERR_SHAPE: invalid rows/cols/seq (cols must be a positive multiple of 256, <= 65536)";
        case Q4K_ERR_ALIGN: return "Q4K_ERR_ALIGN: W, x, X and workspaces must be 16-byte aligned";
        case Q4K_ERR_K: return "Q4K_ERR_K: k must satisfy 1 <= k <= min(rows, 64)";
        case Q4K_ERR_ACT: return "Q4K_ERR_ACT: unknown activation";
        case Q4K_ERR_WORKSPACE: return "Q4K_ERR_WORKSPACE: workspace NULL or too small";
        case Q4K_ERR_ALIAS: return "Q4K_ERR_ALIAS: an output overlaps an input or another output";
        case Q4K_ERR_HIP: return "Q4K_ERR_HIP: HIP runtime error (see q4k_last_hip_error)";
        case Q4K_ERR_EPS: return "Q4K_ERR_EPS: eps must be finite and >= 0";
        case Q4K_ERR_SCRATCH: return "Q4K_ERR_SCRATCH: inter exceeds Q4K_NOALLOC_INTER_MAX (the no-allocation entry point's scratch)";
        default: return "unknown q4k status";
    }
}

Q4K_EXPORT const char *q4k_last_hip_error(void) { return g_last_hip_error; }

Q4K_EXPORT int q4k_matvec(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                          void *stream)
{
    if (!rows_ok(rows) || !cols_ok(cols)) return Q4K_ERR_SHAPE;
    if (rows == 0) return Q4K_OK;
    if (!W || !x || !y) return Q4K_ERR_NULL;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4K_ERR_ALIGN;
    const Span sy = span(y, rows * 4);
    if (overlap(sy, span(W, wbytes(rows, cols))) || overlap(sy, span(x, cols * 4)))
        return Q4K_ERR_ALIAS;
    return finish(q4k::launch_rows_store((const uint8_t *)W, x, y, nullptr, nullptr, rows,
                                             cols, rows, rows, as_stream(stream)), as_stream(stream));
}

Q4K_EXPORT int q6k_matvec(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                          void *stream)
{
    if (!rows_ok(rows) || !cols_ok(cols)) return Q4K_ERR_SHAPE;
    if (rows == 0) return Q4K_OK;
    if (!W || !x || !y) return Q4K_ERR_NULL;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4K_ERR_ALIGN;
    const Span sy = span(y, rows * 4);
    if (overlap(sy, span(W, rows * (cols / Q4K_QK) * Q6K_BLOCK_BYTES)) ||
        overlap(sy, span(x, cols * 4)))
        return Q4K_ERR_ALIAS;
    return finish(q4k::launch_q6k_matvec((const uint8_t *)W, x, y, rows, cols,
                                             as_stream(stream)), as_stream(stream));
}

Q4K_EXPORT int q4k_qkv(const void *Wqkv, const float *x, float *q, float *k, float *v,
                       int64_t q_rows, int64_t kv_rows, int64_t cols, void *stream)
{
    if (q_rows < 0 || kv_rows < 0 || !cols_ok(cols)) return Q4K_ERR_SHAPE;
    const int64_t rows = q_rows + 2 * kv_rows;
    if (!rows_ok(rows)) return Q4K_ERR_SHAPE;
    if (rows == 0) return Q4K_OK;
    if (!Wqkv || !x || (q_rows && !q) || (kv_rows && (!k || !v))) return Q4K_ERR_NULL;
    if (!aligned(Wqkv, 16) || !aligned(x, 16) || !aligned(q, 4) || !aligned(k, 4) ||
        !aligned(v, 4))
        return Q4K_ERR_ALIGN;
    const Span in[2] = {span(Wqkv, wbytes(rows, cols)), span(x, cols * 4)};
    const Span out[3] = {span(q, q_rows * 4), span(k, kv_rows * 4), span(v, kv_rows * 4)};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 2; ++j)
            if (overlap(out[i], in[j])) return Q4K_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(out[i], out[j])) return Q4K_ERR_ALIAS;
    }
    return finish(q4k::launch_rows_store((const uint8_t *)Wqkv, x, q, k, v, rows, cols,
                                             q_rows, q_rows + kv_rows, as_stream(stream)), as_stream(stream));
}

Q4K_EXPORT int q4k_gate_up(const void *Wg, const void *Wu, const float *x, float *h,
                           int64_t inter, int64_t hidden, int act, void *stream)
{
    if (!rows_ok(inter) || !cols_ok(hidden)) return Q4K_ERR_SHAPE;
    if (act != Q4K_ACT_GELU_TANH && act != Q4K_ACT_SILU) return Q4K_ERR_ACT;
    if (inter == 0) return Q4K_OK;
    if (!Wg || !Wu || !x || !h) return Q4K_ERR_NULL;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(x, 16) || !aligned(h, 4))
        return Q4K_ERR_ALIGN;
    const Span sh = span(h, inter * 4);
    if (overlap(sh, span(Wg, wbytes(inter, hidden))) || overlap(sh, span(Wu, wbytes(inter, hidden))) ||
        overlap(sh, span(x, hidden * 4)))
        return Q4K_ERR_ALIAS;
    return finish(q4k::launch_gate_up((const uint8_t *)Wg, (const uint8_t *)Wu, x, h, inter,
                                          hidden, act, as_stream(stream)), as_stream(stream));
}

Q4K_EXPORT size_t q4k_ffn_workspace_bytes(int64_t hidden, int64_t inter)
{
    if (!cols_ok(hidden) || !cols_ok(inter)) return 0;
    return round_up((size_t)inter * 4, 256);
}

Q4K_EXPORT int q4k_ffn(const void *Wg, const void *Wu, const void *Wd, const float *x, float *y,
                       int64_t hidden, int64_t inter, int act, void *ws, size_t ws_bytes,
                       void *stream)
{
    if (!cols_ok(hidden) || !cols_ok(inter)) return Q4K_ERR_SHAPE;
    if (act != Q4K_ACT_GELU_TANH && act != Q4K_ACT_SILU) return Q4K_ERR_ACT;
    if (!Wg || !Wu || !Wd || !x || !y) return Q4K_ERR_NULL;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(x, 16) ||
        !aligned(y, 4))
        return Q4K_ERR_ALIGN;
    const size_t need = q4k_ffn_workspace_bytes(hidden, inter);
    if (!ws || ws_bytes < need) return Q4K_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return Q4K_ERR_ALIGN;
    const Span in[4] = {span(Wg, wbytes(inter, hidden)), span(Wu, wbytes(inter, hidden)),
                        span(Wd, wbytes(hidden, inter)), span(x, hidden * 4)};
    const Span sy = span(y, hidden * 4), sw = span(ws, (int64_t)need);
    if (overlap(sy, sw)) return Q4K_ERR_ALIAS;
    for (int j = 0; j < 4; ++j)
        if (overlap(sy, in[j]) || overlap(sw, in[j])) return Q4K_ERR_ALIAS;
    return finish(q4k::launch_ffn((const uint8_t *)Wg, (const uint8_t *)Wu,
                                      (const uint8_t *)Wd, x, y, hidden, inter, act,
                                      (float *)ws, as_stream(stream)), as_stream(stream));
}

// ------------------------------------------------- no-allocation FFN ---

// The intermediate h of q4k_ffn_noalloc: a file-scope device array, so the
// call needs no workspace and allocates nothing. Each device that runs the
// library holds its own copy until the process ends; every call on a device
// shares that copy (calls that overlap on one device race on it).
static __device__ __align__(256) float scratch[Q4K_NOALLOC_INTER_MAX];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kScratchDevices] = {};

// Device address of the current device's scratch, looked up once per device
// with that device current (host code never passes the array's name itself:
// on the host it is only a stand-in for the symbol).
hipError_t scratch_ptr(float **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

Q4K_EXPORT int q4k_ffn_noalloc(const void *Wg, const void *Wu, const void *Wd, const float *x,
                               float *y, int64_t hidden, int64_t inter, int act, void *stream)
{
    if (!cols_ok(hidden) || !cols_ok(inter)) return Q4K_ERR_SHAPE;
    if (inter > Q4K_NOALLOC_INTER_MAX) return Q4K_ERR_SCRATCH;
    if (act != Q4K_ACT_GELU_TANH && act != Q4K_ACT_SILU) return Q4K_ERR_ACT;
    if (!Wg || !Wu || !Wd || !x || !y) return Q4K_ERR_NULL;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(x, 16) ||
        !aligned(y, 4))
        return Q4K_ERR_ALIGN;
    const Span in[4] = {span(Wg, wbytes(inter, hidden)), span(Wu, wbytes(inter, hidden)),
                        span(Wd, wbytes(hidden, inter)), span(x, hidden * 4)};
    const Span sy = span(y, hidden * 4);
    for (int j = 0; j < 4; ++j)
        if (overlap(sy, in[j])) return Q4K_ERR_ALIAS;
    float *h = nullptr;
    const hipError_t e = scratch_ptr(&h);
    if (e != hipSuccess) return hip_status(e);
    // gate+up writes all of h before the down projection reads it: nothing in
    // the scratch needs clearing between calls
    return finish(q4k::launch_ffn((const uint8_t *)Wg, (const uint8_t *)Wu,
                                  (const uint8_t *)Wd, x, y, hidden, inter, act, h,
                                  as_stream(stream)), as_stream(stream));
}

// ------------------------------------------------ fused residual RMSNorm ---

static bool eps_ok(float eps) { return eps >= 0.0f && eps <= 3.402823466e38f; }  // NaN fails

// Checks shared by the norm entry points: the norm inputs h, delta (optional),
// w (cols floats each) and the optional new stream h_out; `outs` are the
// call's other outputs, `ins` its weights. h_out may overlap nothing.
static int norm_checks(const float *h, const float *delta, const float *w, float eps,
                       float *h_out, int64_t cols, const Span *ins, int nins, const Span *outs,
                       int nouts)
{
    if (!h || !w) return Q4K_ERR_NULL;
    if (!eps_ok(eps)) return Q4K_ERR_EPS;
    if (!aligned(h, 16) || !aligned(delta, 16) || !aligned(w, 16) || !aligned(h_out, 16))
        return Q4K_ERR_ALIGN;
    const Span nin[3] = {span(h, cols * 4), span(delta, delta ? cols * 4 : 0), span(w, cols * 4)};
    const Span so = span(h_out, h_out ? cols * 4 : 0);
    for (int j = 0; j < 3; ++j) {
        if (overlap(so, nin[j])) return Q4K_ERR_ALIAS;
        for (int i = 0; i < nouts; ++i)
            if (overlap(outs[i], nin[j])) return Q4K_ERR_ALIAS;
    }
    for (int j = 0; j < nins; ++j)
        if (overlap(so, ins[j])) return Q4K_ERR_ALIAS;
    for (int i = 0; i < nouts; ++i)
        if (overlap(so, outs[i])) return Q4K_ERR_ALIAS;
    return Q4K_OK;
}

Q4K_EXPORT int q4k_rmsnorm_matvec(const void *W, const float *h, const float *delta,
                                  const float *norm_w, float eps, float *h_out, float *y,
                                  int64_t rows, int64_t cols, void *stream)
{
    if (!rows_ok(rows) || !cols_ok(cols) || rows == 0) return Q4K_ERR_SHAPE;
    if (!W || !y) return Q4K_ERR_NULL;
    if (!aligned(W, 16) || !aligned(y, 4)) return Q4K_ERR_ALIGN;
    const Span sw = span(W, wbytes(rows, cols)), sy = span(y, rows * 4);
    if (overlap(sy, sw)) return Q4K_ERR_ALIAS;
    const int c = norm_checks(h, delta, norm_w, eps, h_out, cols, &sw, 1, &sy, 1);
    if (c != Q4K_OK) return c;
    const q4k::NormIn n = {delta, norm_w, eps, h_out};
    return finish(q4k::launch_rows_store((const uint8_t *)W, h, y, nullptr, nullptr, rows,
                                             cols, rows, rows, as_stream(stream), &n), as_stream(stream));
}

Q4K_EXPORT int q4k_rmsnorm_ffn(const void *Wg, const void *Wu, const void *Wd, const float *h,
                               const float *delta, const float *norm_w, float eps,
                               float *h_out, float *y, int64_t hidden, int64_t inter, int act,
                               void *ws, size_t ws_bytes, void *stream)
{
    if (!cols_ok(hidden) || !cols_ok(inter)) return Q4K_ERR_SHAPE;
    if (act != Q4K_ACT_GELU_TANH && act != Q4K_ACT_SILU) return Q4K_ERR_ACT;
    if (!Wg || !Wu || !Wd || !y) return Q4K_ERR_NULL;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(y, 4))
        return Q4K_ERR_ALIGN;
    const size_t need = q4k_ffn_workspace_bytes(hidden, inter);
    if (!ws || ws_bytes < need) return Q4K_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return Q4K_ERR_ALIGN;
    const Span ins[3] = {span(Wg, wbytes(inter, hidden)), span(Wu, wbytes(inter, hidden)),
                         span(Wd, wbytes(hidden, inter))};
    const Span outs[2] = {span(y, hidden * 4), span(ws, (int64_t)need)};
    if (overlap(outs[0], outs[1])) return Q4K_ERR_ALIAS;
    for (int j = 0; j < 3; ++j)
        if (overlap(outs[0], ins[j]) || overlap(outs[1], ins[j])) return Q4K_ERR_ALIAS;
    const int c = norm_checks(h, delta, norm_w, eps, h_out, hidden, ins, 3, outs, 2);
    if (c != Q4K_OK) return c;
    const q4k::NormIn n = {delta, norm_w, eps, h_out};
    return finish(q4k::launch_ffn((const uint8_t *)Wg, (const uint8_t *)Wu,
                                      (const uint8_t *)Wd, h, y, hidden, inter, act,
                                      (float *)ws, as_stream(stream), &n), as_stream(stream));
}

// lm_head workspace: the per-workgroup candidate lists (k keys of 8 bytes
// each), then the per-workgroup softmax partials (float2).
static size_t lmhead_cand_bytes(int64_t rows, int64_t cols, int k)
{
    return round_up((size_t)q4k::lmhead_max_wgs(rows, cols) * (size_t)k * 8, 256);
}

Q4K_EXPORT int64_t q4k_lmhead_rows_max(int64_t cols)
{
    if (!cols_ok(cols)) return 0;
    return q4k::lmhead_rows_max(cols);
}

// The vocabulary limit, the same test for the workspace size and the calls:
// at most lmhead_rows_max(cols) rows, which keeps the candidate lists within
// what the merge kernel takes.
static bool lmhead_rows_fit(int64_t rows, int64_t cols)
{
    return rows <= q4k::lmhead_rows_max(cols) &&
           q4k::lmhead_max_wgs(rows, cols) <= q4k::kMergeListsMax;
}

Q4K_EXPORT size_t q4k_lmhead_workspace_bytes(int64_t rows, int64_t cols, int k)
{
    if (!rows_ok(rows) || !cols_ok(cols) || rows == 0 || k < 1 || k > Q4K_TOPK_MAX) return 0;
    if (!lmhead_rows_fit(rows, cols)) return 0;
    return lmhead_cand_bytes(rows, cols, k) +
           round_up((size_t)q4k::lmhead_max_wgs(rows, cols) * 8, 256);
}

// Shared by q4k_lmhead_topk (probs == false: top_prob and lse unused) and
// q4k_lmhead_topk_probs.
static int lmhead_call(const void *W, const float *x, float *logits, int64_t rows, int64_t cols,
                       int k, int32_t *top_idx, float *top_val, float *top_prob, float *lse,
                       bool probs, void *ws, size_t ws_bytes, void *stream)
{
    if (!rows_ok(rows) || !cols_ok(cols)) return Q4K_ERR_SHAPE;
    if (k < 1 || k > Q4K_TOPK_MAX || k > rows) return Q4K_ERR_K;
    if (!lmhead_rows_fit(rows, cols)) return Q4K_ERR_SHAPE;
    if (!W || !x || !logits || !top_idx || !top_val) return Q4K_ERR_NULL;
    if (probs && (!top_prob || !lse)) return Q4K_ERR_NULL;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(logits, 4) || !aligned(top_idx, 4) ||
        !aligned(top_val, 4))
        return Q4K_ERR_ALIGN;
    if (probs && (!aligned(top_prob, 4) || !aligned(lse, 4))) return Q4K_ERR_ALIGN;
    const size_t need = q4k_lmhead_workspace_bytes(rows, cols, k);
    if (!ws || ws_bytes < need) return Q4K_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return Q4K_ERR_ALIGN;
    const Span in[2] = {span(W, wbytes(rows, cols)), span(x, cols * 4)};
    const int nout = probs ? 6 : 4;
    const Span out[6] = {span(logits, rows * 4),       span(top_idx, (int64_t)k * 4),
                         span(top_val, (int64_t)k * 4), span(ws, (int64_t)need),
                         span(top_prob, probs ? (int64_t)k * 4 : 0),
                         span(lse, probs ? 4 : 0)};
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < 2; ++j)
            if (overlap(out[i], in[j])) return Q4K_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return Q4K_ERR_ALIAS;
    }
    uint8_t *w8 = (uint8_t *)ws;
    float2 *stats = probs ? (float2 *)(w8 + lmhead_cand_bytes(rows, cols, k)) : nullptr;
    return finish(q4k::launch_lmhead_topk((const uint8_t *)W, x, logits, rows, cols, k,
                                              (uint64_t *)ws, top_idx, top_val, stats,
                                              probs ? top_prob : nullptr, probs ? lse : nullptr,
                                              as_stream(stream)), as_stream(stream));
}

Q4K_EXPORT int q4k_lmhead_topk(const void *W, const float *x, float *logits, int64_t rows,
                               int64_t cols, int k, int32_t *top_idx, float *top_val, void *ws,
                               size_t ws_bytes, void *stream)
{
    return lmhead_call(W, x, logits, rows, cols, k, top_idx, top_val, nullptr, nullptr, false, ws,
                       ws_bytes, stream);
}

Q4K_EXPORT int q4k_lmhead_topk_probs(const void *W, const float *x, float *logits, int64_t rows,
                                     int64_t cols, int k, int32_t *top_idx, float *top_val,
                                     float *top_prob, float *lse, void *ws, size_t ws_bytes,
                                     void *stream)
{
    return lmhead_call(W, x, logits, rows, cols, k, top_idx, top_val, top_prob, lse, true, ws,
                       ws_bytes, stream);
}

Q4K_EXPORT size_t q4k_matmul_workspace_bytes(int64_t rows, int64_t cols, int64_t seq)
{
    if (!rows_ok(rows) || !cols_ok(cols) || seq < 0 || seq > kSeqMax) return 0;
    if (seq < kMfmaMinSeq || rows == 0) return 0;
    return (size_t)q4k::mm_matmul_workspace(rows, cols, seq);
}

Q4K_EXPORT int q4k_matmul(const void *W, const float *X, float *Y, int64_t rows, int64_t cols,
                          int64_t seq, void *ws, size_t ws_bytes, void *stream)
{
    if (!rows_ok(rows) || !cols_ok(cols) || seq < 0 || seq > kSeqMax) return Q4K_ERR_SHAPE;
    if (rows == 0 || seq == 0) return Q4K_OK;
    if (!W || !X || !Y) return Q4K_ERR_NULL;
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, 4)) return Q4K_ERR_ALIGN;
    const size_t need = q4k_matmul_workspace_bytes(rows, cols, seq);
    if (need && (!ws || ws_bytes < need)) return Q4K_ERR_WORKSPACE;
    if (need && !aligned(ws, 16)) return Q4K_ERR_ALIGN;
    const Span sY = span(Y, seq * rows * 4), sw = span(ws, (int64_t)need);
    const Span in[2] = {span(W, wbytes(rows, cols)), span(X, seq * cols * 4)};
    if (overlap(sY, sw)) return Q4K_ERR_ALIAS;
    for (int j = 0; j < 2; ++j)
        if (overlap(sY, in[j]) || overlap(sw, in[j])) return Q4K_ERR_ALIAS;
    hipStream_t s = as_stream(stream);
    if (seq >= kMfmaMinSeq) {
        return finish(q4k::launch_matmul_mfma((const uint8_t *)W, X, Y, rows, cols, seq,
                                                  (uint8_t *)ws, s), as_stream(stream));
    }
    // f32 path: the matvec of every token in one launch (grid row = token;
    // the tokens after the first read W mostly from cache).
    return finish(q4k::launch_rows_store((const uint8_t *)W, X, Y, nullptr, nullptr, rows, cols,
                                             rows, rows, s, nullptr,
                                             q4k::Batch{seq, cols, rows}), as_stream(stream));
}

Q4K_EXPORT size_t q4k_ffn_prefill_workspace_bytes(int64_t seq, int64_t hidden, int64_t inter)
{
    if (seq < 0 || !cols_ok(hidden) || !cols_ok(inter)) return 0;
    // f32 path: h for every token; matrix-core path: its own layout
    size_t need = round_up((size_t)inter * 4 * (size_t)(seq >= 1 && seq < kMfmaMinSeq ? seq : 1), 256);
    if (seq >= kMfmaMinSeq && seq <= kSeqMax) {
        const size_t mm = (size_t)q4k::mm_ffn_workspace(seq, hidden, inter);
        need = mm > need ? mm : need;
    }
    return need;
}

Q4K_EXPORT int q4k_ffn_prefill(const void *Wg, const void *Wu, const void *Wd, const float *X,
                               float *Y, int64_t seq, int64_t hidden, int64_t inter, int act,
                               void *ws, size_t ws_bytes, void *stream)
{
    if (seq < 0 || seq > kSeqMax || !cols_ok(hidden) || !cols_ok(inter)) return Q4K_ERR_SHAPE;
    if (act != Q4K_ACT_GELU_TANH && act != Q4K_ACT_SILU) return Q4K_ERR_ACT;
    if (seq == 0) return Q4K_OK;
    if (!Wg || !Wu || !Wd || !X || !Y) return Q4K_ERR_NULL;
    if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(X, 16) ||
        !aligned(Y, 4))
        return Q4K_ERR_ALIGN;
    const size_t need = q4k_ffn_prefill_workspace_bytes(seq, hidden, inter);
    if (!ws || ws_bytes < need) return Q4K_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return Q4K_ERR_ALIGN;
    const Span in[4] = {span(Wg, wbytes(inter, hidden)), span(Wu, wbytes(inter, hidden)),
                        span(Wd, wbytes(hidden, inter)), span(X, seq * hidden * 4)};
    const Span sY = span(Y, seq * hidden * 4), sw = span(ws, (int64_t)need);
    if (overlap(sY, sw)) return Q4K_ERR_ALIAS;
    for (int j = 0; j < 4; ++j)
        if (overlap(sY, in[j]) || overlap(sw, in[j])) return Q4K_ERR_ALIAS;
    hipStream_t s = as_stream(stream);
    if (seq >= kMfmaMinSeq) {
        return finish(q4k::launch_ffn_prefill_mfma((const uint8_t *)Wg, (const uint8_t *)Wu,
                                                       (const uint8_t *)Wd, X, Y, seq, hidden,
                                                       inter, act, (uint8_t *)ws, s), as_stream(stream));
    }
    // f32 path: gate+up for every token in one launch, then down likewise
    return finish(q4k::launch_ffn((const uint8_t *)Wg, (const uint8_t *)Wu,
                                      (const uint8_t *)Wd, X, Y, hidden, inter, act, (float *)ws,
                                      s, nullptr, seq), as_stream(stream));
}

// ------------------------------------------------------ measurement helpers ---

static bool probe_launch_ok(int grid, int threads)
{
    return grid >= 1 && grid <= 65536 && threads >= 64 && threads <= 1024 && threads % 64 == 0;
}

Q4K_EXPORT int q4k_probe_read(const void *buf, int64_t bytes, int grid, int threads, int depth,
                              int contiguous, uint32_t *sink, void *stream)
{
    if (bytes < 16 || bytes % 16 != 0 || bytes >= ((int64_t)1 << 31) ||
        !probe_launch_ok(grid, threads) ||
        (depth != 1 && depth != 2 && depth != 4 && depth != 8 && depth != 16))
        return Q4K_ERR_SHAPE;
    if (!buf || !sink) return Q4K_ERR_NULL;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return Q4K_ERR_ALIGN;
    if (overlap(span(sink, 4), span(buf, bytes))) return Q4K_ERR_ALIAS;
    return finish(q4k::launch_probe_read((const uint8_t *)buf, bytes, grid, threads, depth,
                                         contiguous != 0, sink, as_stream(stream)),
                  as_stream(stream));
}

Q4K_EXPORT int q4k_probe_empty(int grid, int threads, uint32_t *sink, void *stream)
{
    if (!probe_launch_ok(grid, threads)) return Q4K_ERR_SHAPE;
    if (!sink) return Q4K_ERR_NULL;
    if (!aligned(sink, 4)) return Q4K_ERR_ALIGN;
    return finish(q4k::launch_probe_empty(grid, threads, sink, as_stream(stream)),
                  as_stream(stream));
}
