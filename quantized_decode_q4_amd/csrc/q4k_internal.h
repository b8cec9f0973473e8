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

// Row-streaming kernels (q4k_rows.hip).
// y rows [0, split0) -> o0, [split0, split1) -> o1, [split1, rows) -> o2.
hipError_t launch_rows_store(const uint8_t *W, const float *x, float *o0, float *o1, float *o2,
                             int64_t rows, int64_t cols, int64_t split0, int64_t split1,
                             hipStream_t s);
hipError_t launch_gate_up(const uint8_t *Wg, const uint8_t *Wu, const float *x, float *h,
                          int64_t rows, int64_t cols, int act, hipStream_t s);
// lm_head: number of candidate-producing workgroups for a shape (device independent).
int64_t lmhead_num_wgs(int64_t rows, int64_t cols);
hipError_t launch_lmhead_topk(const uint8_t *W, const float *x, float *logits, int64_t rows,
                              int64_t cols, int k, uint64_t *cand, int32_t *top_idx,
                              float *top_val, hipStream_t s);

}  // namespace q4k
