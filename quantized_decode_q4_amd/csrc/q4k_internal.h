// Internal launch interface between the C ABI (q4k_api.hip) and the kernel
// translation units. Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

constexpr int kQK = 256;          // weights per super-block
constexpr int kBlockBytes = 144;  // bytes per super-block
constexpr int kTopkMax = 64;
constexpr int kColsMax = 65536;
constexpr int kLmheadRowsPerWgMax = 4096;
constexpr int kMergeListsMax = 1024;    // per-workgroup candidate lists the merge takes

// Block-floating-point activation planes of n activations (n a multiple of
// 256) as staged in LDS: three byte planes of n bytes, then n/32 scales and
// n/32 sums (f32).
__host__ __device__ constexpr int64_t planes_bytes(int64_t n) { return 3 * n + n / 4; }

// Residual RMSNorm fused into a projection's input: the activations become
// s * w with s = x + delta (delta may be null) and the outputs are scaled by
// 1/sqrt(mean(s^2) + eps); h_out (may be null) receives s.
struct NormIn {
    const float *delta;
    const float *w;
    float eps;
    float *h_out;
};

// Row-streaming kernels (q4k_rows.hip).
// A batch of nvec activation vectors in one launch: vector v reads
// x + v * x_stride and writes o0 + v * o_stride (no norm, no o1/o2 split).
struct Batch {
    int64_t nvec = 1;
    int64_t x_stride = 0;
    int64_t o_stride = 0;
};
// y rows [0, split0) -> o0, [split0, split1) -> o1, [split1, rows) -> o2.
hipError_t launch_rows_store(const uint8_t *W, const float *x, float *o0, float *o1, float *o2,
                             int64_t rows, int64_t cols, int64_t split0, int64_t split1,
                             hipStream_t s, const NormIn *norm = nullptr, const Batch &bt = Batch{});
hipError_t launch_gate_up(const uint8_t *Wg, const uint8_t *Wu, const float *x, float *h,
                          int64_t rows, int64_t cols, int act, hipStream_t s,
                          const NormIn *norm = nullptr, const Batch &bt = Batch{});
// Gated FFN: gate+up with the activation applied (h, f32[inter]), then the
// down projection reading h. A norm applies to the gate+up input. nvec > 1
// (no norm): x [nvec][hidden], h [nvec][inter], y [nvec][hidden].
hipError_t launch_ffn(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const float *x,
                      float *y, int64_t hidden, int64_t inter, int act, float *h, hipStream_t s,
                      const NormIn *norm = nullptr, int64_t nvec = 1);
// Q6_K matvec (GGUF Q6_K rows, 210 bytes per 256 weights): y = W x.
hipError_t launch_q6k_matvec(const uint8_t *W, const float *x, float *y, int64_t rows,
                             int64_t cols, hipStream_t s);
// lm_head: candidate-producing workgroups used on this device, and the most
// any device uses for the shape (sizes the workspace).
int64_t lmhead_num_wgs(int64_t rows, int64_t cols);
int64_t lmhead_max_wgs(int64_t rows, int64_t cols);
// Largest rows for which lmhead_max_wgs stays within kMergeListsMax.
int64_t lmhead_rows_max(int64_t cols);
// With stats (lmhead_max_wgs float2 partials), also the softmax over all
// rows: lse[0] and top_prob[k]; stats == nullptr skips both.
hipError_t launch_lmhead_topk(const uint8_t *W, const float *x, float *logits, int64_t rows,
                              int64_t cols, int k, uint64_t *cand, int32_t *top_idx,
                              float *top_val, float2 *stats, float *top_prob, float *lse,
                              hipStream_t s);

// Matrix-core prefill (q4k_mm.hip), for seq >= 64 tokens. Workspace sizes
// (bytes) for the current device, and the launches that carve them.
int64_t mm_matmul_workspace(int64_t rows, int64_t cols, int64_t seq);
int64_t mm_ffn_workspace(int64_t seq, int64_t hidden, int64_t inter);
// Y[seq][rows] = X W^T.
hipError_t launch_matmul_mfma(const uint8_t *W, const float *X, float *Y, int64_t rows,
                              int64_t cols, int64_t seq, uint8_t *ws, hipStream_t s);
// Gated FFN for seq tokens: H = act(X Wg^T) * (X Wu^T) (bf16), Y = H Wd^T.
hipError_t launch_ffn_prefill_mfma(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd,
                                   const float *X, float *Y, int64_t seq, int64_t hidden,
                                   int64_t inter, int act, uint8_t *ws, hipStream_t s);

// Measurement helpers (q4k_probe.hip): a streaming read of bytes (a multiple
// of 16, below 2^31) at buf with 128-bit buffer loads, grid x threads, depth
// loads in flight per thread (1, 2, 4, 8 or 16), grid-stride or one contiguous
// range per workgroup; and an empty kernel of grid x threads.
hipError_t launch_probe_read(const uint8_t *buf, int64_t bytes, int grid, int threads, int depth,
                             bool contiguous, uint32_t *sink, hipStream_t s);
hipError_t launch_probe_empty(int grid, int threads, uint32_t *sink, hipStream_t s);

}  // namespace q4k
