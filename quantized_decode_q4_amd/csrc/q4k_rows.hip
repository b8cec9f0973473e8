// Row-streaming Q4_K kernels for decode (one activation vector):
//   matvec / fused QKV, fused gate+up with the gated activation, and the
//   lm_head matvec with a per-workgroup top-k plus a single-workgroup merge.
//
// Sources: infer-compute README, "Shaders" table (q4k_matvec, q4k_qkv_proj,
// q4k_ffn_gate_up, geglu_gelu_tanh / geglu_silu) and "Key Optimizations"
// table (wide loads, several rows per thread group, fused gate+up);
// Performance -- infer-inference, "Honest Path Breakdown" (lm_head logits on
// the GPU) and the infer-inference README Overview example (top-5).
//
// Work decomposition (gfx950, wave64):
//  * A row of cols = 256*nb weights is nb super-blocks. Each block splits into
//    four 32-byte "units": unit g holds quant bytes 32g..32g+31, i.e. all 32
//    weights of sub-block 2g (low nibbles) and of sub-block 2g+1 (high
//    nibbles). A row has U = 4*nb units.
//  * Thread t of a workgroup owns unit u = t / RPS of rows r = t % RPS of every
//    sweep: the workgroup covers RPS consecutive rows per sweep and walks its
//    contiguous row range. The thread keeps the 64 activations of its unit in
//    registers for the whole kernel (loaded once, reused for every row), so
//    the activation is read from memory once per thread, not once per row.
//  * Per row the thread loads 2 x 16 B of quants and the 16 B block header
//    (d, dmin, packed 6-bit scales/mins) with 128-bit loads; a wave covers
//    64/RPS consecutive units of RPS rows, so each load instruction reads
//    contiguous runs of every row.
//  * Partial dot products are reduced across the 64/RPS units of a wave with
//    xor shuffles, then across waves through LDS, in a fixed order (results
//    are deterministic; no atomics).
//  * Dequantisation uses w = d*sc*q - dmin*m per 32-weight sub-block s:
//      sum_j w_j x_j = d*sc_s*sum_j q_j x_j - dmin*m_s*sum_j x_j,
//    so the min term needs only the per-thread activation sums.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_internal.h"

namespace q4k {
namespace {

enum Epi { EPI_STORE = 0, EPI_GATE_UP = 1, EPI_LOGITS = 2 };

struct RowsArgs {
    const uint8_t *W0;
    const uint8_t *W1;
    const float *x;
    float *o0;
    float *o1;
    float *o2;
    uint64_t *cand;
    int64_t rows;
    int64_t split0;
    int64_t split1;
    int64_t rows_per_wg;
    int32_t nb;
    int32_t U;
    int32_t act;
    int32_t k;
};

__device__ __forceinline__ float act_apply(float z, int act)
{
    if (act == 0) {
        const float c = 0.7978845608028654f;  // sqrt(2/pi)
        return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
    }
    return z / (1.0f + expf(-z));
}

// Partial dot product of one unit (sub-blocks A = 2g and B = 2g+1 of a block)
// of one row with the thread's 64 activations.
//   nq[0..7]: the 32 quant bytes; hd: the 16-byte block header.
// Low nibbles are A's quants; high nibbles are kept in place (16*q) and the
// factor 1/16 is folded into B's scale (exact, a power of two).
__device__ __forceinline__ uint32_t and_opaque(uint32_t v, uint32_t m)
{
    // An AND the optimiser cannot see through: the byte conversions below then
    // stay single v_cvt_f32_ubyte{0..3} instructions instead of a bit-field
    // extract followed by a conversion.
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(m), "v"(v));
    return r;
}

__device__ __forceinline__ float unit_dot(const uint32_t (&nq)[8], uint4 hd,
                                          const float (&xa)[32], const float (&xb)[32],
                                          float SA, float SB, int sh, bool upper)
{
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t lo = and_opaque(nq[k], 0x0F0F0F0Fu);
        const uint32_t hi = and_opaque(nq[k], 0xF0F0F0F0u);
        a0 = fmaf((float)(lo & 0xFFu), xa[4 * k + 0], a0);
        a1 = fmaf((float)((lo >> 8) & 0xFFu), xa[4 * k + 1], a1);
        a0 = fmaf((float)((lo >> 16) & 0xFFu), xa[4 * k + 2], a0);
        a1 = fmaf((float)(lo >> 24), xa[4 * k + 3], a1);
        b0 = fmaf((float)(hi & 0xFFu), xb[4 * k + 0], b0);
        b1 = fmaf((float)((hi >> 8) & 0xFFu), xb[4 * k + 1], b1);
        b0 = fmaf((float)((hi >> 16) & 0xFFu), xb[4 * k + 2], b0);
        b1 = fmaf((float)(hi >> 24), xb[4 * k + 3], b1);
    }
    const float d = __half2float(__ushort_as_half((unsigned short)(hd.x & 0xFFFFu)));
    const float dmin = __half2float(__ushort_as_half((unsigned short)(hd.x >> 16)));
    // Scale bytes: hd.y = s[0..3], hd.z = s[4..7], hd.w = s[8..11].
    // Sub-blocks 0..3: sc = s[j] & 63, m = s[j+4] & 63.
    // Sub-blocks 4..7: sc = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
    //                  m  = (s[j+4] >> 4) | (s[j]   >> 6) << 4.
    // This unit needs the byte pair starting at 2*(g&1) (shift sh = 16*(g&1)).
    const uint32_t sc_src = upper ? hd.w : hd.y;
    const uint32_t m_src = upper ? (hd.w >> 4) : hd.z;
    const uint32_t low_mask = upper ? 0x0F0Fu : 0x3F3Fu;
    const uint32_t top_mask = upper ? 0x3030u : 0u;
    const uint32_t sc2 = ((sc_src >> sh) & low_mask) | ((hd.y >> (sh + 2)) & top_mask);
    const uint32_t m2 = ((m_src >> sh) & low_mask) | ((hd.z >> (sh + 2)) & top_mask);
    const float scA = (float)(sc2 & 0xFFu);
    const float scB = (float)((sc2 >> 8) & 0xFFu) * 0.0625f;
    const float mA = (float)(m2 & 0xFFu);
    const float mB = (float)((m2 >> 8) & 0xFFu);
    const float t1 = fmaf(scA, a0 + a1, scB * (b0 + b1));
    const float t2 = fmaf(mA, SA, mB * SB);
    return fmaf(d, t1, -dmin * t2);
}

// Orderable 64-bit key of a (logit, row) pair: larger key = earlier in the
// top-k order (value descending, then index ascending). NaN maps to the
// lowest value class (high word 0); key 0 itself means "no candidate".
__device__ __forceinline__ uint64_t topk_key(float v, uint32_t idx)
{
    uint32_t hi;
    if (v != v) {
        hi = 0u;
    } else {
        if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
        const uint32_t b = __float_as_uint(v);
        hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
    return ((uint64_t)hi << 32) | (uint64_t)(~idx);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off)
{
    const uint32_t lo = __shfl_xor((unsigned int)(v & 0xFFFFFFFFu), off);
    const uint32_t hi = __shfl_xor((unsigned int)(v >> 32), off);
    return ((uint64_t)hi << 32) | lo;
}

// Workgroup-wide maximum of a 64-bit key (all threads get the result).
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t *scratch)
{
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = shfl_xor_u64(v, off);
        v = o > v ? o : v;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nwaves = (blockDim.x + 63) >> 6;
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    uint64_t m = 0;
    for (int w = 0; w < nwaves; ++w) m = scratch[w] > m ? scratch[w] : m;
    __syncthreads();
    return m;
}

// Unconditional 16-byte loads through a bounds-checked buffer resource: an
// offset at or beyond the resource's size reads zeros instead of faulting, so
// lanes with nothing to load (rows past the end, unused units) issue the same
// instructions as the others. Every path then has the same number of loads in
// flight, which keeps the in-order wait counts of the software pipeline exact.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// One in-flight row-unit per matrix: 32 quant bytes + the 16-byte header.
template <int NMAT>
struct Slot {
    uint32_t q[NMAT][8];
    uint4 h[NMAT];
};

// off: byte offset of the row's block header inside the workgroup's resource
// (kOutOfRange for nothing); qoff = 16 + 32g, the unit's quant bytes.
template <int NMAT>
__device__ __forceinline__ void load_slot(Slot<NMAT> &sl, const __amdgpu_buffer_rsrc_t (&rs)[NMAT],
                                          uint32_t off, uint32_t qoff)
{
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        sl.h[m] = bload16(rs[m], off);
        const uint4 q0 = bload16(rs[m], off + qoff);
        const uint4 q1 = bload16(rs[m], off + qoff + 16);
        sl.q[m][0] = q0.x; sl.q[m][1] = q0.y; sl.q[m][2] = q0.z; sl.q[m][3] = q0.w;
        sl.q[m][4] = q1.x; sl.q[m][5] = q1.y; sl.q[m][6] = q1.z; sl.q[m][7] = q1.w;
    }
}

// Persistent row-streaming kernel.
//  RPS  rows per sweep (threads t = u*RPS + r own unit u of row r of a sweep)
//  NMAT 1 (one matrix) or 2 (gate and up rows sharing the activation)
//  EPI  epilogue: store / gated activation / logits + block top-k
//  D    sweeps whose loads are in flight while one sweep is computed
// Workgroup w processes the contiguous sweeps [S*w/G, S*(w+1)/G) of the
// S = ceil(rows / RPS) sweeps. The quant/header loads of the first D sweeps
// are issued before the activation slice, then every step issues sweep i+D
// and computes sweep i (a register ring of D+1 slots, statically indexed by
// unrolling). Wave partial sums go to an LDS bank; every FB sweeps one barrier
// publishes them and threads t < FB*RPS finish the rows.
template <int RPS, int NMAT, int EPI, int MAXT, int D>
__global__ __launch_bounds__(MAXT) void rows_kernel(RowsArgs a)
{
    static_assert(RPS >= 1 && RPS <= 64 && (64 % RPS) == 0, "RPS must divide 64");
    constexpr int NW = MAXT / 64;
    constexpr int FB = 8;
    __shared__ float red[2][NW][FB * NMAT * RPS];
    __shared__ float lg[EPI == EPI_LOGITS ? kLmheadRowsPerWgMax : 1];
    __shared__ uint8_t taken[EPI == EPI_LOGITS ? kLmheadRowsPerWgMax : 1];
    __shared__ uint64_t keys_scratch[EPI == EPI_LOGITS ? NW : 1];

    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int nwaves = blockDim.x >> 6;
    const int u = t / RPS;
    const int r = t % RPS;
    const bool uact = u < a.U;
    const int b = u >> 2, g = u & 3;
    const int sh = (g & 1) * 16;
    const bool upper = g >= 2;
    const int64_t rowbytes = (int64_t)a.nb * kBlockBytes;
    const int64_t unit_off = (int64_t)b * kBlockBytes;
    const int64_t S = (a.rows + RPS - 1) / RPS;
    const int64_t s_begin = S * blockIdx.x / gridDim.x;
    const int64_t s_end = S * (blockIdx.x + 1) / gridDim.x;
    const int64_t row_begin = s_begin * RPS;
    const int64_t row_stop = min(s_end * RPS, a.rows);

    // Buffer resources over this workgroup's rows (the host keeps the span
    // below 2^31 bytes); offsets are relative to row_begin.
    __amdgpu_buffer_rsrc_t rs[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
        rs[m] = make_rsrc((m == 0 ? a.W0 : a.W1) + row_begin * rowbytes,
                          (uint32_t)((row_stop - row_begin) * rowbytes));
    const uint32_t qoff = 16u + 32u * (uint32_t)g;
    // byte offset of (sweep s, this thread's row) or kOutOfRange
    auto slot_off = [&](int64_t sw) -> uint32_t {
        const int64_t row = sw * RPS + r;
        return (uact && row < row_stop) ? (uint32_t)((row - row_begin) * rowbytes + unit_off)
                                        : kOutOfRange;
    };

    Slot<NMAT> buf[D + 1];
#pragma unroll
    for (int j = 0; j < D; ++j) load_slot<NMAT>(buf[j], rs, slot_off(s_begin + j), qoff);

    // The thread's 64 activations: x[256b + 64g + 0..31] (sub-block A) and
    // x[256b + 64g + 32..63] (sub-block B), loaded once.
    // Unused units read zeros (out-of-range offset).
    float xa[32], xb[32];
    float SA = 0.f, SB = 0.f;
    {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)a.nb * 1024u);
        const uint32_t xo = uact ? (uint32_t)(256 * b + 64 * g) * 4u : kOutOfRange;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 va = bload16(rx, xo + 16u * i);
            const uint4 vb = bload16(rx, xo + 128u + 16u * i);
            xa[4 * i + 0] = __uint_as_float(va.x); xa[4 * i + 1] = __uint_as_float(va.y);
            xa[4 * i + 2] = __uint_as_float(va.z); xa[4 * i + 3] = __uint_as_float(va.w);
            xb[4 * i + 0] = __uint_as_float(vb.x); xb[4 * i + 1] = __uint_as_float(vb.y);
            xb[4 * i + 2] = __uint_as_float(vb.z); xb[4 * i + 3] = __uint_as_float(vb.w);
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            SA += xa[i];
            SB += xb[i];
        }
    }

    int kb = 0, bank = 0;
    for (int64_t s = s_begin; s < s_end; s += D + 1) {
#pragma unroll
        for (int j = 0; j <= D; ++j) {
            const int64_t sj = s + j;
            if (sj >= s_end) break;  // uniform
            // the next sweep's loads go out before this sweep is computed;
            // past the end they read zeros (unused)
            if (D > 0) load_slot<NMAT>(buf[(j + D) % (D + 1)], rs, slot_off(sj + D), qoff);
            if (D == 0) load_slot<NMAT>(buf[0], rs, slot_off(sj), qoff);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                float v = unit_dot(buf[j].q[m], buf[j].h[m], xa, xb, SA, SB, sh, upper);
#pragma unroll
                for (int off = RPS; off < 64; off <<= 1) v += __shfl_xor(v, off);
                if (lane < RPS) red[bank][wave][(kb * NMAT + m) * RPS + lane] = v;
            }
            ++kb;
            if (kb == FB || sj == s_end - 1) {
                __syncthreads();
                if (t < kb * RPS) {
                    const int k = t / RPS, rr = t % RPS;
                    const int64_t row = (sj - kb + 1 + k) * RPS + rr;
                    if (row < row_stop) {
                        float v0 = 0.f, v1 = 0.f;
                        for (int w = 0; w < nwaves; ++w) {
                            v0 += red[bank][w][(k * NMAT + 0) * RPS + rr];
                            if (NMAT == 2) v1 += red[bank][w][(k * NMAT + 1) * RPS + rr];
                        }
                        if (EPI == EPI_STORE) {
                            if (row < a.split0)
                                a.o0[row] = v0;
                            else if (row < a.split1)
                                a.o1[row - a.split0] = v0;
                            else
                                a.o2[row - a.split1] = v0;
                        } else if (EPI == EPI_GATE_UP) {
                            a.o0[row] = act_apply(v0, a.act) * v1;
                        } else {
                            a.o0[row] = v0;
                            lg[row - row_begin] = v0;
                            taken[row - row_begin] = 0;
                        }
                    }
                }
                kb = 0;
                bank ^= 1;
            }
        }
    }

    if (EPI == EPI_LOGITS) {
        // Per-workgroup top-k of its rows, written in rank order: k rounds of
        // a workgroup-wide max over orderable keys; the winner is removed.
        __syncthreads();
        const int n = (int)(row_stop - row_begin);
        uint64_t *out = a.cand + (int64_t)blockIdx.x * a.k;
        for (int round = 0; round < a.k; ++round) {
            uint64_t best = 0;
            for (int j = t; j < n; j += blockDim.x) {
                if (taken[j]) continue;
                const uint64_t kk = topk_key(lg[j], (uint32_t)(row_begin + j));
                best = kk > best ? kk : best;
            }
            const uint64_t win = block_max_u64(best, keys_scratch);
            if (t == 0) {
                out[round] = win;
                if (win != 0) taken[(int64_t)(~(uint32_t)(win & 0xFFFFFFFFu)) - row_begin] = 1;
            }
            __syncthreads();
        }
    }
}

// Merge of the per-workgroup candidate lists (each sorted in rank order) into
// the global top-k: a k-way merge. Thread t owns lists t, t+256, ...; each
// round the workgroup takes the largest list head and that list advances.
constexpr int kMergeThreads = 256;
constexpr int kMergeListsPerThread = 4;   // up to 1024 lists

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(const uint64_t *cand, int nlists,
                                                                    int k, const float *logits,
                                                                    int32_t *top_idx,
                                                                    float *top_val)
{
    __shared__ uint64_t scratch[kMergeThreads / 64];
    const int t = threadIdx.x;
    int pos[kMergeListsPerThread];
    uint64_t head[kMergeListsPerThread];
#pragma unroll
    for (int i = 0; i < kMergeListsPerThread; ++i) {
        const int l = t + i * kMergeThreads;
        pos[i] = 0;
        head[i] = l < nlists ? cand[(int64_t)l * k] : 0ull;
    }
    for (int round = 0; round < k; ++round) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kMergeListsPerThread; ++i) best = head[i] > best ? head[i] : best;
        const uint64_t win = block_max_u64(best, scratch);
        if (win != 0) {
#pragma unroll
            for (int i = 0; i < kMergeListsPerThread; ++i) {
                if (head[i] == win) {  // keys are unique (they embed the row)
                    const int l = t + i * kMergeThreads;
                    ++pos[i];
                    head[i] = pos[i] < k ? cand[(int64_t)l * k + pos[i]] : 0ull;
                }
            }
        }
        if (t == 0) {
            if (win == 0) {
                top_idx[round] = -1;
                top_val[round] = __uint_as_float(0x7FC00000u);
            } else {
                const uint32_t idx = ~(uint32_t)(win & 0xFFFFFFFFu);
                top_idx[round] = (int32_t)idx;
                top_val[round] = logits[idx];
            }
        }
    }
}

// ---------------------------------------------------------------- host ---

struct Shape {
    int rps;
    int threads;
};

Shape pick_shape(int64_t cols)
{
    const int U = (int)(cols / kQK) * 4;
    int rps = 1;
    while (U * rps < 256 && rps < 64) rps *= 2;
    const int threads = ((U * rps + 63) / 64) * 64;
    return {rps, threads};
}

// Compute units of the current device (cached per device).
int device_cus()
{
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Workgroups of `threads` threads resident per CU for a kernel using ~vgprs
// registers per lane (512 per SIMD lane, 4 SIMDs, wave64).
int wgs_per_cu(int threads, int vgprs)
{
    const int waves_per_simd = 512 / vgprs;
    const int waves = (threads + 63) / 64;
    const int per_cu = (4 * waves_per_simd) / waves;
    return per_cu < 1 ? 1 : per_cu;
}

template <int NMAT, int EPI, int D>
hipError_t launch_rows(const RowsArgs &a, int rps, int threads, int64_t nwg, hipStream_t s)
{
    const dim3 grid((unsigned)nwg), block((unsigned)threads);
    if (threads > 512) {
        // only reachable with one row per sweep (cols > 32768)
        hipLaunchKernelGGL((rows_kernel<1, NMAT, EPI, 1024, 0>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    switch (rps) {
#define Q4K_RPS_CASE(R) \
    case R: hipLaunchKernelGGL((rows_kernel<R, NMAT, EPI, 512, D>), grid, block, 0, s, a); break;
        Q4K_RPS_CASE(1)
        Q4K_RPS_CASE(2)
        Q4K_RPS_CASE(4)
        Q4K_RPS_CASE(8)
        Q4K_RPS_CASE(16)
        Q4K_RPS_CASE(32)
        Q4K_RPS_CASE(64)
#undef Q4K_RPS_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

RowsArgs base_args(int64_t rows, int64_t cols)
{
    RowsArgs a{};
    a.rows = rows;
    a.nb = (int32_t)(cols / kQK);
    a.U = a.nb * 4;
    a.split0 = rows;
    a.split1 = rows;
    return a;
}

// Persistent grid: as many workgroups as fit on the device at once, never
// more than there are sweeps, and enough that one workgroup's rows span less
// than 2^30 bytes (its buffer resource uses 32-bit offsets).
int64_t grid_for(int64_t rows, int64_t cols, const Shape &sh, int vgprs)
{
    const int64_t S = (rows + sh.rps - 1) / sh.rps;
    int64_t g = (int64_t)device_cus() * wgs_per_cu(sh.threads, vgprs);
    const int64_t sweep_bytes = (int64_t)sh.rps * (cols / kQK) * kBlockBytes;
    const int64_t max_sweeps = ((int64_t)1 << 30) / sweep_bytes;   // >= 1 for cols <= 65536
    const int64_t min_g = (S + max_sweeps - 2) / (max_sweeps - 1 > 0 ? max_sweeps - 1 : 1);
    if (g < min_g) g = min_g;
    return S < g ? S : g;
}

constexpr int kVgprStore = 168;   // budget the kernels are written to (3 waves/SIMD)
constexpr int kLmheadWgs = 512;   // device-independent: fixes the workspace size

}  // namespace

hipError_t launch_rows_store(const uint8_t *W, const float *x, float *o0, float *o1, float *o2,
                             int64_t rows, int64_t cols, int64_t split0, int64_t split1,
                             hipStream_t s)
{
    RowsArgs a = base_args(rows, cols);
    a.W0 = W;
    a.x = x;
    a.o0 = o0;
    a.o1 = o1;
    a.o2 = o2;
    a.split0 = split0;
    a.split1 = split1;
    const Shape sh = pick_shape(cols);
    return launch_rows<1, EPI_STORE, 3>(a, sh.rps, sh.threads, grid_for(rows, cols, sh, kVgprStore), s);
}

hipError_t launch_gate_up(const uint8_t *Wg, const uint8_t *Wu, const float *x, float *h,
                          int64_t rows, int64_t cols, int act, hipStream_t s)
{
    RowsArgs a = base_args(rows, cols);
    a.W0 = Wg;
    a.W1 = Wu;
    a.x = x;
    a.o0 = h;
    a.act = act;
    const Shape sh = pick_shape(cols);
    return launch_rows<2, EPI_GATE_UP, 1>(a, sh.rps, sh.threads, grid_for(rows, cols, sh, kVgprStore),
                                          s);
}

int64_t lmhead_num_wgs(int64_t rows, int64_t cols)
{
    const Shape sh = pick_shape(cols);
    const int64_t S = (rows + sh.rps - 1) / sh.rps;
    // enough workgroups that each holds at most kLmheadRowsPerWgMax rows
    int64_t g = kLmheadWgs;
    const int64_t min_g = (S * sh.rps + kLmheadRowsPerWgMax - 1) / (kLmheadRowsPerWgMax - sh.rps);
    if (g < min_g) g = min_g;
    return S < g ? S : g;
}

hipError_t launch_lmhead_topk(const uint8_t *W, const float *x, float *logits, int64_t rows,
                              int64_t cols, int k, uint64_t *cand, int32_t *top_idx,
                              float *top_val, hipStream_t s)
{
    RowsArgs a = base_args(rows, cols);
    a.W0 = W;
    a.x = x;
    a.o0 = logits;
    a.cand = cand;
    a.k = k;
    const Shape sh = pick_shape(cols);
    const int64_t nwg = lmhead_num_wgs(rows, cols);
    hipError_t e = launch_rows<1, EPI_LOGITS, 3>(a, sh.rps, sh.threads, nwg, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(1), dim3(kMergeThreads), 0, s, cand, (int)nwg, k,
                       logits, top_idx, top_val);
    return hipGetLastError();
}

}  // namespace q4k
