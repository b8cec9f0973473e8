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
__device__ __forceinline__ float unit_dot(const uint32_t (&nq)[8], uint4 hd,
                                          const float (&xa)[32], const float (&xb)[32],
                                          float SA, float SB, int sh, bool upper)
{
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t lo = nq[k] & 0x0F0F0F0Fu;
        const uint32_t hi = nq[k] & 0xF0F0F0F0u;
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

template <int RPS, int P, int NMAT, int EPI, int MAXT>
__global__ __launch_bounds__(MAXT) void rows_kernel(RowsArgs a)
{
    static_assert(RPS >= 1 && RPS <= 64 && (64 % RPS) == 0, "RPS must divide 64");
    constexpr int NW = MAXT / 64;
    __shared__ float red[NW][P * NMAT * RPS];
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
    const int64_t row_begin = (int64_t)blockIdx.x * a.rows_per_wg;
    const int64_t row_end = min(row_begin + a.rows_per_wg, a.rows);

    // The thread's 64 activations: x[256b + 64g + 0..31] (sub-block A) and
    // x[256b + 64g + 32..63] (sub-block B).
    float xa[32], xb[32];
    float SA = 0.f, SB = 0.f;
    if (uact) {
        const float4 *xp = reinterpret_cast<const float4 *>(a.x + 256 * b + 64 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 va = xp[i];
            const float4 vb = xp[8 + i];
            xa[4 * i + 0] = va.x; xa[4 * i + 1] = va.y; xa[4 * i + 2] = va.z; xa[4 * i + 3] = va.w;
            xb[4 * i + 0] = vb.x; xb[4 * i + 1] = vb.y; xb[4 * i + 2] = vb.z; xb[4 * i + 3] = vb.w;
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            SA += xa[i];
            SB += xb[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) xa[i] = xb[i] = 0.f;
    }

    const int64_t unit_off = (int64_t)b * kBlockBytes;
    for (int64_t s0 = row_begin; s0 < row_end; s0 += (int64_t)P * RPS) {
        uint32_t nq[P][NMAT][8];
        uint4 hd[P][NMAT];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int64_t row = s0 + p * RPS + r;
            const bool ok = uact && row < row_end;
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                if (ok) {
                    const uint8_t *base = (m == 0 ? a.W0 : a.W1) + row * rowbytes + unit_off;
                    hd[p][m] = *reinterpret_cast<const uint4 *>(base);
                    const uint4 q0 = *reinterpret_cast<const uint4 *>(base + 16 + 32 * g);
                    const uint4 q1 = *reinterpret_cast<const uint4 *>(base + 32 + 32 * g);
                    nq[p][m][0] = q0.x; nq[p][m][1] = q0.y; nq[p][m][2] = q0.z; nq[p][m][3] = q0.w;
                    nq[p][m][4] = q1.x; nq[p][m][5] = q1.y; nq[p][m][6] = q1.z; nq[p][m][7] = q1.w;
                } else {
                    hd[p][m] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                    for (int i = 0; i < 8; ++i) nq[p][m][i] = 0u;
                }
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (s0 + p * RPS >= row_end) break;  // uniform: empty batch slot
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                float v = unit_dot(nq[p][m], hd[p][m], xa, xb, SA, SB, sh, upper);
#pragma unroll
                for (int off = RPS; off < 64; off <<= 1) v += __shfl_xor(v, off);
                if (lane < RPS) red[wave][(p * NMAT + m) * RPS + lane] = v;
            }
        }
        __syncthreads();
        if (t < P * RPS) {
            const int p = t / RPS, rr = t % RPS;
            const int64_t row = s0 + p * RPS + rr;
            if (row < row_end) {
                float v0 = 0.f, v1 = 0.f;
                for (int w = 0; w < nwaves; ++w) {
                    v0 += red[w][(p * NMAT + 0) * RPS + rr];
                    if (NMAT == 2) v1 += red[w][(p * NMAT + 1) * RPS + rr];
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
        __syncthreads();
    }

    if (EPI == EPI_LOGITS) {
        // Per-workgroup top-k of rows [row_begin, row_end): k rounds of a
        // workgroup-wide max over orderable keys; the winner is removed.
        const int n = (int)(row_end - row_begin);
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

// Single-workgroup merge of nc candidate keys into the global top-k.
constexpr int kMergeThreads = 1024;
constexpr int kMergePerThread = kMergeCandMax / kMergeThreads;

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(const uint64_t *cand, int nc,
                                                                    int k, const float *logits,
                                                                    int32_t *top_idx,
                                                                    float *top_val)
{
    __shared__ uint64_t scratch[kMergeThreads / 64];
    const int t = threadIdx.x;
    uint64_t mine[kMergePerThread];
#pragma unroll
    for (int i = 0; i < kMergePerThread; ++i) {
        const int c = t + i * kMergeThreads;
        mine[i] = c < nc ? cand[c] : 0ull;
    }
    for (int round = 0; round < k; ++round) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kMergePerThread; ++i) best = mine[i] > best ? mine[i] : best;
        const uint64_t win = block_max_u64(best, scratch);
        if (win != 0) {
#pragma unroll
            for (int i = 0; i < kMergePerThread; ++i)
                if (mine[i] == win) mine[i] = 0ull;
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

template <int P, int NMAT, int EPI>
hipError_t launch_rows(const RowsArgs &a, int rps, int threads, int64_t nwg, hipStream_t s)
{
    const dim3 grid((unsigned)nwg), block((unsigned)threads);
    if (threads > 512) {
        // only reachable with one row per sweep (cols > 32768)
        hipLaunchKernelGGL((rows_kernel<1, 1, NMAT, EPI, 1024>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    switch (rps) {
#define Q4K_RPS_CASE(R) \
    case R: hipLaunchKernelGGL((rows_kernel<R, P, NMAT, EPI, 512>), grid, block, 0, s, a); break;
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

// Rows per workgroup: whole sweeps of rps rows, aiming at about target
// workgroups.
int64_t rows_per_wg_for(int64_t rows, int rps, int64_t target_wgs)
{
    int64_t per = (rows + target_wgs - 1) / target_wgs;
    per = (per + rps - 1) / rps * rps;
    if (per < rps) per = rps;
    return per;
}

}  // namespace

hipError_t launch_rows_store(const uint8_t *W, const float *x, float *o0, float *o1, float *o2,
                             int64_t rows, int64_t cols, int64_t split0, int64_t split1,
                             hipStream_t s)
{
    constexpr int P = 4;
    RowsArgs a = base_args(rows, cols);
    a.W0 = W;
    a.x = x;
    a.o0 = o0;
    a.o1 = o1;
    a.o2 = o2;
    a.split0 = split0;
    a.split1 = split1;
    const Shape sh = pick_shape(cols);
    a.rows_per_wg = rows_per_wg_for(rows, sh.rps, 1024);
    const int64_t nwg = (rows + a.rows_per_wg - 1) / a.rows_per_wg;
    return launch_rows<P, 1, EPI_STORE>(a, sh.rps, sh.threads, nwg, s);
}

hipError_t launch_gate_up(const uint8_t *Wg, const uint8_t *Wu, const float *x, float *h,
                          int64_t rows, int64_t cols, int act, hipStream_t s)
{
    constexpr int P = 2;
    RowsArgs a = base_args(rows, cols);
    a.W0 = Wg;
    a.W1 = Wu;
    a.x = x;
    a.o0 = h;
    a.act = act;
    const Shape sh = pick_shape(cols);
    a.rows_per_wg = rows_per_wg_for(rows, sh.rps, 1024);
    const int64_t nwg = (rows + a.rows_per_wg - 1) / a.rows_per_wg;
    return launch_rows<P, 2, EPI_GATE_UP>(a, sh.rps, sh.threads, nwg, s);
}

int64_t lmhead_num_wgs(int64_t rows, int64_t cols)
{
    const Shape sh = pick_shape(cols);
    int64_t per = rows_per_wg_for(rows, sh.rps, 512);
    if (per > kLmheadRowsPerWgMax) per = kLmheadRowsPerWgMax;
    return (rows + per - 1) / per;
}

hipError_t launch_lmhead_topk(const uint8_t *W, const float *x, float *logits, int64_t rows,
                              int64_t cols, int k, uint64_t *cand, int32_t *top_idx,
                              float *top_val, hipStream_t s)
{
    constexpr int P = 4;
    RowsArgs a = base_args(rows, cols);
    a.W0 = W;
    a.x = x;
    a.o0 = logits;
    a.cand = cand;
    a.k = k;
    const Shape sh = pick_shape(cols);
    int64_t per = rows_per_wg_for(rows, sh.rps, 512);
    if (per > kLmheadRowsPerWgMax) per = kLmheadRowsPerWgMax;
    a.rows_per_wg = per;
    const int64_t nwg = (rows + per - 1) / per;
    hipError_t e = launch_rows<P, 1, EPI_LOGITS>(a, sh.rps, sh.threads, nwg, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(1), dim3(kMergeThreads), 0, s, cand,
                       (int)(nwg * k), k, logits, top_idx, top_val);
    return hipGetLastError();
}

}  // namespace q4k
