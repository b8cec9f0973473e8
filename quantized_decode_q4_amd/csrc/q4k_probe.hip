// Measurement helpers: the streaming-read ceiling and the cost of a launch on
// this part, made with the same unconditional 128-bit buffer loads as the
// decode kernels (out-of-range lanes read zeros). They are the device-side
// counterparts of the pages' bandwidth and raw-dispatch profiles
// (infer-compute README, "Benchmarks: Profile (bottleneck analysis)") and
// take no part in the decode path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ uint4 probe_load(__amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Every load's data is folded into acc; the store happens only for a value
// the random-looking fold never produces in practice, so the loads stay.
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

// Grid stride: thread g of the grid reads the 16 bytes at (i * G * T + g) * 16
// for i = 0, 1, ...; DEPTH loads are issued before their data is used.
template <int DEPTH>
__global__ __launch_bounds__(1024) void read_gstride_kernel(const uint8_t *buf, uint32_t bytes,
                                                            uint32_t *sink)
{
    const auto rs = probe_rsrc(buf, bytes);
    // 64-bit offsets: grid * threads * 16 * DEPTH can exceed 2^32; offsets at
    // or past the end are clamped to it (the resource reads zeros there)
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 16u;
    uint32_t acc = 0;
    for (uint64_t off = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16u; off < bytes;
         off += DEPTH * stride) {
        uint4 v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const uint64_t o = off + d * stride;
            v[d] = probe_load(rs, (uint32_t)(o < bytes ? o : bytes));
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    if (acc == kSinkMagic) sink[0] = acc;
}

// Contiguous ranges: workgroup w reads its own 16-byte-aligned share of the
// buffer, blockDim * 16 bytes per load instruction, DEPTH in flight.
template <int DEPTH>
__global__ __launch_bounds__(1024) void read_contig_kernel(const uint8_t *buf, uint32_t bytes,
                                                           uint32_t *sink)
{
    uint64_t per = ((uint64_t)bytes + gridDim.x - 1) / gridDim.x;
    per = (per + 15) & ~(uint64_t)15;
    const uint64_t lo = (uint64_t)blockIdx.x * per;
    const uint64_t hi = lo + per < bytes ? lo + per : bytes;
    if (lo >= hi) return;
    const auto rs = probe_rsrc(buf + lo, (uint32_t)(hi - lo));
    const uint64_t n = hi - lo, step = (uint64_t)blockDim.x * 16u;
    uint32_t acc = 0;
    for (uint64_t off = threadIdx.x * 16u; off < n; off += DEPTH * step) {
        uint4 v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const uint64_t o = off + d * step;
            v[d] = probe_load(rs, (uint32_t)(o < n ? o : n));
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    if (acc == kSinkMagic) sink[0] = acc;
}

__global__ void empty_kernel(uint32_t *sink)
{
    if (threadIdx.x == 0xFFFFFu) sink[0] = 0;   // never true: an empty body
}

}  // namespace

hipError_t launch_probe_read(const uint8_t *buf, int64_t bytes, int grid, int threads, int depth,
                             bool contiguous, uint32_t *sink, hipStream_t s)
{
    const dim3 g((unsigned)grid), b((unsigned)threads);
    const uint32_t n = (uint32_t)bytes;
#define Q4K_PROBE_CASE(DD)                                                                   \
    case DD:                                                                                 \
        if (contiguous)                                                                      \
            hipLaunchKernelGGL(read_contig_kernel<DD>, g, b, 0, s, buf, n, sink);            \
        else                                                                                 \
            hipLaunchKernelGGL(read_gstride_kernel<DD>, g, b, 0, s, buf, n, sink);           \
        break;
    switch (depth) {
        Q4K_PROBE_CASE(1)
        Q4K_PROBE_CASE(2)
        Q4K_PROBE_CASE(4)
        Q4K_PROBE_CASE(8)
        Q4K_PROBE_CASE(16)
        default: return hipErrorInvalidValue;
    }
#undef Q4K_PROBE_CASE
    return hipGetLastError();
}

hipError_t launch_probe_empty(int grid, int threads, uint32_t *sink, hipStream_t s)
{
    hipLaunchKernelGGL(empty_kernel, dim3((unsigned)grid), dim3((unsigned)threads), 0, s, sink);
    return hipGetLastError();
}

}  // namespace q4k
