// Row-streaming Q4_K kernels for decode (one activation vector):
//   matvec / fused QKV, fused gate+up with the gated activation, and the
//   lm_head matvec with a per-workgroup top-k plus a k-way merge.
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
//    nibbles). A row has U = 4*nb units; unit u covers columns 64u..64u+63.
//  * Thread t of a workgroup owns unit u = t / RPS of rows r = t % RPS of every
//    sweep (RPS consecutive rows). The workgroup walks a contiguous range of
//    sweeps (a persistent grid), keeping D sweeps of loads in flight while it
//    computes one (a register ring). The thread's activations stay in
//    registers for the whole kernel.
//  * Per row the thread reads 2 x 16 B of quants and the 16 B block header
//    with unconditional bounds-checked buffer loads.
//  * Partial dot products are reduced across the 64/RPS units of a wave with
//    xor shuffles, then across waves through LDS, in a fixed order (results
//    are deterministic; no atomics).
//
// Arithmetic. w = d*sc_s*q - dmin*m_s per 32-weight sub-block s, so
//     sum_j w_j x_j = d*sc_s*sum_j q_j x_j - dmin*m_s*sum_j x_j.
// The activations of each sub-block are held in block floating point:
//     x_j = X_s * (p0_j + 256 p1_j + 65536 p2_j),  X_s = 2^(e_s - 22),
// with max_j |x_j| < 2^e_s, p0, p1 unsigned bytes and p2 a signed byte (the
// two's-complement bytes of a 24-bit integer |x_int| <= 2^22; rounding error
// <= 2^-23 of the sub-block maximum, the resolution of f32 at that maximum).
// sum_j q_j x_j is then three byte dot products (v_dot4_u32_u8 for p0, p1,
// v_dot4_i32_i8 for p2) on the raw nibbles, exact in 32-bit integers, scaled
// by X_s once per sub-block. The min term uses the f32 sum of the sub-block's
// activations. Non-finite activations make X_s NaN (outputs become NaN).
// The rounding error of an activation is below 2^-22 of its sub-block's
// largest magnitude. A sub-block is held this way only when that magnitude is
// at most kBfpSpread times the mean magnitude of its 32 activations, so every
// activation is represented to within 2^-22 * 6 = 1.4e-6 of the sub-block's
// mean magnitude. A wave whose units cover a sub-block beyond that spread (an
// outlier activation) runs the whole launch with f32 multiply-adds instead.
//
// Q6_K (the other K-quant of the Shaders table, q6k_matvec; GGUF block of
// 210 bytes: ql[128], qh[64], 16 signed scales, f16 d) runs through the same
// kernel with FMT_Q6K: unit g = 2n + h of a block holds the 64 weights
// 128n + 32j + 16h + i (j = 0..3, i = 0..15), whose low nibbles are ql bytes
// 64n + 16h + i (j = 0, 2) and 64n + 32 + 16h + i (j = 1, 3) and whose high
// bit pairs are qh bytes 32n + 16h + i. Blocks are only 2-byte aligned, so each
// field is read with 4-byte-aligned loads one dword wider and realigned in
// registers (v_alignbyte); d is read with a 2-byte load, so no load reaches
// past its block. Activations are f32: sum_i w_i x_i over a 16-weight
// sub-block is d*sc*(sum_i q_i x_i - 32 sum_i x_i).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "q4k_internal.h"

// Launch tunables, chosen by timing sweeps on MI355X (1, 2, 3, 4, 8
// workgroups per CU; 0 to 3 sweeps in flight): one persistent workgroup per
// CU and one sweep in flight were best or within 2% of best for every shape
// of the decode step.
#ifndef Q4K_ROWS_FB
#define Q4K_ROWS_FB 8               // sweeps per cross-wave reduction batch
#endif
#ifndef Q4K_LMHEAD_FB
#define Q4K_LMHEAD_FB 4             // the same for lm_head (64 sweeps per workgroup at 262144 rows)
#endif
#ifndef Q4K_STORE_D
#define Q4K_STORE_D 1               // sweeps in flight, block-floating-point matvec
#endif
#ifndef Q4K_F32_DEEP_SWEEPS
#define Q4K_F32_DEEP_SWEEPS 4       // f32 launches: two sweeps in flight from this many per workgroup
#endif
#ifndef Q4K_STORE_WGS_PER_CU
#define Q4K_STORE_WGS_PER_CU 1
#endif
#ifndef Q4K_STORE_F32_SWEEPS
#define Q4K_STORE_F32_SWEEPS 2      // sweeps per workgroup (x 8/RPS) up to which matvec uses f32 activations
#endif
#ifndef Q4K_GATE_UP_D
#define Q4K_GATE_UP_D 1
#endif
#ifndef Q4K_GATE_UP_WGS_PER_CU
#define Q4K_GATE_UP_WGS_PER_CU 1
#endif
#ifndef Q4K_GATE_UP_SPLIT
#define Q4K_GATE_UP_SPLIT 1         // gate and up rows in two wave groups (where both fit)
#endif
#ifndef Q4K_DOWN_WGS_PER_CU
#define Q4K_DOWN_WGS_PER_CU 1
#endif
#ifndef Q4K_PRE_SWEEPS
#define Q4K_PRE_SWEEPS 1            // sweeps issued before the activations are prepared
#endif
#ifndef Q4K_INTERLEAVE
#define Q4K_INTERLEAVE 1            // long launches: workgroups take every G-th sweep
#endif
#ifndef Q4K_WAVE_LOCAL_X
#define Q4K_WAVE_LOCAL_X 1          // each wave converts the activations its own units use
#endif
#ifndef Q4K_DPP_QUAD
#define Q4K_DPP_QUAD 1              // quad max/sum of the conversion with DPP instead of LDS permutes
#endif
#ifndef Q6K_D
#define Q6K_D 1                     // sweeps in flight, Q6_K matvec
#endif
#ifndef Q6K_WGS_PER_CU
#define Q6K_WGS_PER_CU 1
#endif
#ifndef Q4K_LMHEAD_D
#define Q4K_LMHEAD_D 1
#endif
#ifndef Q4K_LMHEAD_WGS_PER_CU
#define Q4K_LMHEAD_WGS_PER_CU 2
#endif
#ifndef Q4K_LMHEAD_WIDE
#define Q4K_LMHEAD_WIDE 1           // lm_head: one workgroup per CU, twice the rows per sweep
#endif

namespace q4k {
namespace {

enum Epi { EPI_STORE = 0, EPI_GATE_UP = 1, EPI_LOGITS = 3 };
// How the thread holds its 64 activations:
//  XS_LDS    block floating point, converted through LDS (byte dot
//            products): without a fused norm each wave converts the groups its
//            own units read, with one the whole workgroup converts together
//  XS_THREAD block floating point, each thread converts its own 64 (rows too
//            wide for the LDS copy)
//  XS_F32    plain f32 in registers (f32 multiply-adds). Used where a thread
//            computes only a few rows, so that no conversion has to be paid
//            for: the down projection of the FFN.
enum XSrc { XS_LDS = 0, XS_THREAD = 1, XS_F32 = 3 };
// Weight format of the rows.
enum Fmt { FMT_Q4K = 0, FMT_Q6K = 1 };
constexpr int kQ6Bytes = 210;   // bytes per Q6_K super-block
// Rows up to this many columns stage the normalised activations in LDS when a
// norm is fused into an f32-activation launch (cols * 4 bytes and the padding).
constexpr int64_t kNormLdsCols = 8192;
// Sweeps per workgroup from which a launch interleaves its sweeps.
constexpr int64_t kIlvMinSweeps = 8;

__host__ __device__ constexpr int fmt_block_bytes(int fmt) { return fmt == FMT_Q6K ? kQ6Bytes : kBlockBytes; }

struct RowsArgs {
    const uint8_t *W0;
    const uint8_t *W1;
    const float *x;
    float *o0;
    float *o1;
    float *o2;
    uint64_t *cand;          // EPI_LOGITS
    float2 *stats;           // EPI_LOGITS, optional: per-workgroup (max, sum of exp(l - max))
    // Fused residual RMSNorm of the input (nw != nullptr): s = x + delta (delta
    // optional), activations s * nw, every output scaled by
    // 1/sqrt(mean(s^2) + eps); workgroup 0 writes s to h_out (optional).
    const float *delta;
    const float *nw;
    float *h_out;
    float eps;
    int64_t rows;
    int64_t split0;
    int64_t split1;
    int32_t nb;
    int32_t U;
    int32_t act;
    int32_t k;
    // Sweeps per workgroup, set by the launch: sq each, and one more for the
    // first srem workgroups (sq * gridDim.x + srem sweeps in all).
    int32_t sq;
    int32_t srem;
    int32_t nwg;             // gridDim.x
    int32_t nthr;            // blockDim.x
    int32_t xpass;           // (cols / 8 + nthr - 1) / nthr: passes of a workgroup-wide conversion
    int32_t ilv;             // 1: workgroup w takes sweeps w, w+G, w+2G, ... (else a contiguous range)
    // Several activation vectors in one launch (grid row y = vector y): x
    // and o0 advance by these many floats per vector (o1, o2 unused then).
    int64_t x_stride;
    int64_t o_stride;
};

// Every kernel argument in scalar registers at once, at the top of the
// kernel: the compiler otherwise loads each field where a branch first needs
// it, and each such load is another memory round trip (the argument block of
// a launch is cold) ahead of the first weight load.
__device__ __forceinline__ void args_to_sgprs(const RowsArgs &a)
{
    asm volatile("" ::"s"(a.W0), "s"(a.W1), "s"(a.x), "s"(a.o0), "s"(a.o1), "s"(a.o2),
                 "s"(a.cand), "s"(a.stats), "s"(a.delta), "s"(a.nw), "s"(a.h_out), "s"(a.eps),
                 "s"(a.rows), "s"(a.split0), "s"(a.split1), "s"(a.nb), "s"(a.U), "s"(a.act),
                 "s"(a.k), "s"(a.sq), "s"(a.srem), "s"(a.nwg), "s"(a.nthr), "s"(a.xpass), "s"(a.ilv),
                 "s"(a.x_stride), "s"(a.o_stride));
}

// Slot of 16-byte chunk i of an f32 activation row staged in LDS. A unit's 64
// activations are 16 chunks (256 bytes, one pass over the LDS banks), and the
// threads of a wave read chunk c of consecutive units together: each unit is
// followed by one chunk of padding, so that those reads fall on different
// banks instead of all on the same four (a 32-way conflict for two rows per
// sweep). Unit u then starts at slot 17u.
__device__ __forceinline__ int xslot(int i) { return i + (i >> 4); }
constexpr int64_t kXPadNum = 17, kXPadDen = 16;   // padded size: cols * 4 * 17 / 16 bytes

__device__ __forceinline__ float act_apply(float z, int act)
{
    if (act == 0) {
        const float c = 0.7978845608028654f;  // sqrt(2/pi)
        return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
    }
    return z / (1.0f + expf(-z));
}

// ---------------------------------------------------------------- loads ---

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

// Q6_K: one in-flight row-unit per matrix, as loaded (4-byte aligned, one
// dword wider than each field): ql of quarters 0/2 and 1/3 and qh (5 dwords
// each), the 8 scale bytes of the half (3 dwords), d (16 bits), and the byte
// misalignment of the block (0 or 2).
template <int NMAT>
struct Slot6 {
    uint32_t q[NMAT][15];
    uint32_t sc[NMAT][3];
    uint32_t d[NMAT];
    uint32_t mis;
};

__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0);
}

// off: byte offset of the block inside the (4-byte aligned) resource, or
// kOutOfRange; n, h: the unit's half and 16-byte slice.
template <int NMAT>
__device__ __forceinline__ void load_slot6(Slot6<NMAT> &sl, const __amdgpu_buffer_rsrc_t (&rs)[NMAT],
                                           uint32_t off, int n, int h)
{
    const uint32_t mis = off & 3u;      // 0 or 2 (blocks start at even bytes)
    const uint32_t o = off - mis;       // kOutOfRange stays out of range
    const uint32_t fa = o + 64u * n + 16u * h, fb = fa + 32u, fh = o + 128u + 32u * n + 16u * h;
    const uint32_t fs = o + 192u + 8u * n;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const uint4 a = bload16(rs[m], fa);
        const uint4 b = bload16(rs[m], fb);
        const uint4 c = bload16(rs[m], fh);
        sl.q[m][0] = a.x; sl.q[m][1] = a.y; sl.q[m][2] = a.z; sl.q[m][3] = a.w;
        sl.q[m][4] = bload4(rs[m], fa + 16u);
        sl.q[m][5] = b.x; sl.q[m][6] = b.y; sl.q[m][7] = b.z; sl.q[m][8] = b.w;
        sl.q[m][9] = bload4(rs[m], fb + 16u);
        sl.q[m][10] = c.x; sl.q[m][11] = c.y; sl.q[m][12] = c.z; sl.q[m][13] = c.w;
        sl.q[m][14] = bload4(rs[m], fh + 16u);
        const auto sv = __builtin_amdgcn_raw_buffer_load_b64(rs[m], (int)fs, 0, 0);
        sl.sc[m][0] = sv[0];
        sl.sc[m][1] = sv[1];
        sl.sc[m][2] = bload4(rs[m], fs + 8u);
        sl.d[m] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs[m], (int)(off + 208u), 0, 0);
    }
    sl.mis = mis;
}

// ------------------------------------------------ block floating point ---

// Largest magnitude of a sub-block held in block floating point, in units of
// its mean magnitude (see the arithmetic note at the top).
#ifndef Q4K_BFP_SPREAD
#define Q4K_BFP_SPREAD 6.0f
#endif
constexpr float kBfpSpread = Q4K_BFP_SPREAD;

// Whether 32 activations with largest magnitude amax and magnitude sum abssum
// are within that spread (all zeros are).
__device__ __forceinline__ bool bfp_spread_ok(float amax, float abssum)
{
    return 32.0f * amax <= kBfpSpread * abssum;
}

// Shift taking the sub-block to 22-bit integers and the scale back; the
// maximum magnitude amax and the f32 sum (NaN/Inf detector) are given.
__device__ __forceinline__ void bfp_params(float amax, float sum, int &shift, float &X)
{
    const int e = __builtin_amdgcn_frexp_expf(amax);   // amax < 2^e
    shift = 22 - e;
    X = __builtin_amdgcn_ldexpf(1.0f, e - 22);
    if (amax == 0.0f) {
        shift = 0;
        X = 0.0f;
    }
    if (!(fabsf(sum) <= 3.402823466e38f) || !(amax <= 3.402823466e38f))
        X = __int_as_float(0x7FC00000);
}

__device__ __forceinline__ int to_int22(float v, int shift)
{
    return (int)__builtin_rintf(__builtin_amdgcn_ldexpf(v, shift));
}

// Bytes 0, 1, 2 of four 24-bit integers a, b, c, d, transposed into plane
// dwords: P0 = [a.b0 b.b0 c.b0 d.b0], P1 = [.. b1 ..], P2 = [.. b2 ..].
__device__ __forceinline__ void pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                      uint32_t &P0, uint32_t &P1, uint32_t &P2)
{
    const uint32_t u01 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
    const uint32_t u23 = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
    P0 = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
    P1 = __builtin_amdgcn_perm(u23, u01, 0x07060302u);
    P2 = __builtin_amdgcn_perm(b, a, 0x0c0c0602u) | __builtin_amdgcn_perm(d, c, 0x06020c0cu);
}

// The thread's 64 activations (sub-blocks A = 2u and B = 2u+1), in one of two
// forms sharing the same registers:
//  block floating point: r[8 pl + k] is dword k of plane pl of A, r[24 + 8 pl
//    + k] the same of B, r[48..51] = X_A, X_B, S_A, S_B (scales, f32 sums);
//  f32 (waves outside the block-floating-point spread): r[0..31] = A,
//    r[32..63] = B, r[64], r[65] = S_A, S_B.
struct XUnit {
    float r[66];
};

// Convert 32 f32 activations into planes (per-thread path): planes to
// p[0..23] as in XUnit, scale X, sum S; false when the sub-block is beyond
// the block-floating-point spread.
__device__ __forceinline__ bool planes32(const float (&v)[32], float *p, float &X, float &S)
{
    float amax = 0.f, sum = 0.f, abssum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        amax = fmaxf(amax, fabsf(v[i]));
        sum += v[i];
        abssum += fabsf(v[i]);
    }
    int shift;
    bfp_params(amax, sum, shift, X);
    S = sum;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint32_t p0, p1, p2;
        pack4((uint32_t)to_int22(v[4 * k], shift), (uint32_t)to_int22(v[4 * k + 1], shift),
              (uint32_t)to_int22(v[4 * k + 2], shift), (uint32_t)to_int22(v[4 * k + 3], shift),
              p0, p1, p2);
        p[k] = __uint_as_float(p0);
        p[8 + k] = __uint_as_float(p1);
        p[16 + k] = __uint_as_float(p2);
    }
    return bfp_spread_ok(amax, abssum);
}

// ------------------------------------------------------------ compute ---

// Partial dot product of one unit of one row with the thread's activations.
__device__ __forceinline__ float unit_dot(const uint32_t (&nq)[8], uint4 hd, const XUnit &xu,
                                          int sh, bool upper)
{
    uint32_t a0 = 0u, a1 = 0u, b0 = 0u, b1 = 0u;
    int a2 = 0, b2 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t lo = nq[k] & 0x0F0F0F0Fu;          // sub-block A quants
        const uint32_t hi = (nq[k] >> 4) & 0x0F0F0F0Fu;   // sub-block B quants
        a0 = __builtin_amdgcn_udot4(lo, __float_as_uint(xu.r[k]), a0, false);
        a1 = __builtin_amdgcn_udot4(lo, __float_as_uint(xu.r[8 + k]), a1, false);
        a2 = __builtin_amdgcn_sdot4((int)lo, (int)__float_as_uint(xu.r[16 + k]), a2, false);
        b0 = __builtin_amdgcn_udot4(hi, __float_as_uint(xu.r[24 + k]), b0, false);
        b1 = __builtin_amdgcn_udot4(hi, __float_as_uint(xu.r[32 + k]), b1, false);
        b2 = __builtin_amdgcn_sdot4((int)hi, (int)__float_as_uint(xu.r[40 + k]), b2, false);
    }
    // a0 + 256 a1 < 2^25 fits in 32 bits exactly
    const float gA = fmaf(65536.0f, (float)a2, (float)(a0 + (a1 << 8)));
    const float gB = fmaf(65536.0f, (float)b2, (float)(b0 + (b1 << 8)));

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
    const float scB = (float)((sc2 >> 8) & 0xFFu);
    const float mA = (float)(m2 & 0xFFu);
    const float mB = (float)((m2 >> 8) & 0xFFu);
    const float t1 = fmaf(scA * xu.r[48], gA, (scB * xu.r[49]) * gB);
    const float t2 = fmaf(mA, xu.r[50], mB * xu.r[51]);
    return fmaf(d, t1, -dmin * t2);
}

// An AND the optimiser cannot see through: the byte conversions of the f32
// path then stay single v_cvt_f32_ubyte{0..3} instructions instead of a
// bit-field extract followed by a conversion.
__device__ __forceinline__ uint32_t and_opaque(uint32_t v, uint32_t m)
{
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(m), "v"(v));
    return r;
}

// f32 path: the thread's 64 activations and their sub-block sums.
struct XF32 {
    float xa[32], xb[32];
    float SA, SB;
};

// Partial dot product of one unit of one row, f32 multiply-adds. Low nibbles
// are A's quants; high nibbles are kept in place (16q) and the factor 1/16 is
// folded into B's scale (exact, a power of two). xa, xb: the 32 activations
// of sub-blocks A and B; SA, SB their sums.
__device__ __forceinline__ float unit_dot_f32p(const uint32_t (&nq)[8], uint4 hd, const float *xa,
                                               const float *xb, float SA, float SB, int sh,
                                               bool upper)
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

__device__ __forceinline__ float unit_dot_f32(const uint32_t (&nq)[8], uint4 hd, const XF32 &xf,
                                              int sh, bool upper)
{
    return unit_dot_f32p(nq, hd, xf.xa, xf.xb, xf.SA, xf.SB, sh, upper);
}

// The same on the f32 view of an XUnit.
__device__ __forceinline__ float unit_dot_f32u(const uint32_t (&nq)[8], uint4 hd, const XUnit &xu,
                                               int sh, bool upper)
{
    return unit_dot_f32p(nq, hd, xu.r, xu.r + 32, xu.r[64], xu.r[65], sh, upper);
}

// Q6_K partial dot product of one unit of one row, f32 multiply-adds. The
// thread's 64 activations are xf.xa = quarters 0, 1 and xf.xb = quarters 2,
// 3 (16 each); s6[j] is the sum of quarter j's activations.
__device__ __forceinline__ float unit_dot_q6(const uint32_t (&q)[15], const uint32_t (&sc)[3],
                                             uint32_t dbits, uint32_t mis, const XF32 &xf,
                                             const float (&s6)[4], int h)
{
    const uint32_t sh = mis;   // bytes to drop: 0 or 2
    uint32_t qa[4], qb[4], qh[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        qa[k] = __builtin_amdgcn_alignbyte(q[k + 1], q[k], sh);
        qb[k] = __builtin_amdgcn_alignbyte(q[k + 6], q[k + 5], sh);
        qh[k] = __builtin_amdgcn_alignbyte(q[k + 11], q[k + 10], sh);
    }
    float acc[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j][0] = acc[j][1] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // six-bit quants of quarters 0..3 for l = 16h + 4k + c, c = byte
        const uint32_t q0 = and_opaque(qa[k], 0x0F0F0F0Fu) | ((qh[k] << 4) & 0x30303030u);
        const uint32_t q1 = and_opaque(qb[k], 0x0F0F0F0Fu) | ((qh[k] << 2) & 0x30303030u);
        const uint32_t q2 = and_opaque(qa[k] >> 4, 0x0F0F0F0Fu) | (qh[k] & 0x30303030u);
        const uint32_t q3 = and_opaque(qb[k] >> 4, 0x0F0F0F0Fu) | ((qh[k] >> 2) & 0x30303030u);
        const uint32_t qj[4] = {q0, q1, q2, q3};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float *xj = j < 2 ? &xf.xa[16 * j] : &xf.xb[16 * (j - 2)];
            acc[j][0] = fmaf((float)(qj[j] & 0xFFu), xj[4 * k + 0], acc[j][0]);
            acc[j][1] = fmaf((float)((qj[j] >> 8) & 0xFFu), xj[4 * k + 1], acc[j][1]);
            acc[j][0] = fmaf((float)((qj[j] >> 16) & 0xFFu), xj[4 * k + 2], acc[j][0]);
            acc[j][1] = fmaf((float)(qj[j] >> 24), xj[4 * k + 3], acc[j][1]);
        }
    }
    // scales of quarters j: bytes h + 2j of the half's 8 scale bytes
    const uint32_t s03 = __builtin_amdgcn_alignbyte(sc[1], sc[0], sh);
    const uint32_t s47 = __builtin_amdgcn_alignbyte(sc[2], sc[1], sh);
    const int hs = 8 * h;
    const float sc0 = (float)(int8_t)((s03 >> hs) & 0xFFu);
    const float sc1 = (float)(int8_t)((s03 >> (hs + 16)) & 0xFFu);
    const float sc2 = (float)(int8_t)((s47 >> hs) & 0xFFu);
    const float sc3 = (float)(int8_t)((s47 >> (hs + 16)) & 0xFFu);
    float t = sc0 * fmaf(-32.f, s6[0], acc[0][0] + acc[0][1]);
    t = fmaf(sc1, fmaf(-32.f, s6[1], acc[1][0] + acc[1][1]), t);
    t = fmaf(sc2, fmaf(-32.f, s6[2], acc[2][0] + acc[2][1]), t);
    t = fmaf(sc3, fmaf(-32.f, s6[3], acc[3][0] + acc[3][1]), t);
    const float d = __half2float(__ushort_as_half((unsigned short)(dbits & 0xFFFFu)));
    return d * t;
}

// ------------------------------------------------------ wave reduction ---

// Sum over the lanes of a wave that are congruent modulo RPS (every lane gets
// its class's sum). Within 16-lane rows a cyclic rotation by `off` pairs lane
// i with i+off (mod 16), which is all a sum needs; across rows the gfx950
// permlane swaps exchange rows (16) and halves (32): v_permlane32_swap x, y
// swaps the upper half of x with the lower half of y, so with x = y = v the
// two registers add up to v + v[lane ^ 32] (likewise for 16-lane rows). No
// LDS traffic, unlike a shuffle through ds_bpermute.
// The swaps are written as inline asm: with the builtin, this compiler folds
// the sum of the two results of a swap of equal inputs into twice the first
// result (a miscompile found on MI355X; the asm form was checked there
// against a CPU sum for every RPS).
template <int RPS>
__device__ __forceinline__ float wave_sum_mod(float v)
{
    if (RPS <= 1) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
    if (RPS <= 2) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
    if (RPS <= 4) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    if (RPS <= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    if (RPS <= 16) {
        float x = v, y = v;
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
        v = x + y;
    }
    if (RPS <= 32) {
        float x = v, y = v;
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
        v = x + y;
    }
    return v;
}

// ---------------------------------------------------------------- top-k ---

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

// The logit a key was made from (the NaN class decodes to a NaN; -0 was
// folded into +0).
__device__ __forceinline__ float topk_key_value(uint64_t key)
{
    const uint32_t hi = (uint32_t)(key >> 32);
    return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint64_t join_u64(uint32_t hi, uint32_t lo)
{
    return ((uint64_t)hi << 32) | lo;
}

// Largest 64-bit key over the 64 lanes of a wave (every lane gets it), in
// the same pattern as wave_sum_mod: rotations by 1, 2, 4, 8 inside 16-lane
// rows, then the row and half swaps (inline asm, see wave_sum_mod).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#define Q4K_ROR_MAX(C)                                                                     \
    {                                                                                      \
        const uint64_t o = join_u64(dpp_u32<C>((uint32_t)(v >> 32)), dpp_u32<C>((uint32_t)v)); \
        v = o > v ? o : v;                                                                 \
    }
    Q4K_ROR_MAX(0x121)
    Q4K_ROR_MAX(0x122)
    Q4K_ROR_MAX(0x124)
    Q4K_ROR_MAX(0x128)
#undef Q4K_ROR_MAX
    {
        uint32_t xl = (uint32_t)v, yl = xl, xh = (uint32_t)(v >> 32), yh = xh;
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(xl), "+v"(yl));
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(xh), "+v"(yh));
        const uint64_t a = join_u64(xh, xl), b = join_u64(yh, yl);
        v = a > b ? a : b;
    }
    {
        uint32_t xl = (uint32_t)v, yl = xl, xh = (uint32_t)(v >> 32), yh = xh;
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(xl), "+v"(yl));
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(xh), "+v"(yh));
        const uint64_t a = join_u64(xh, xl), b = join_u64(yh, yl);
        v = a > b ? a : b;
    }
    return v;
}

// Largest 32-bit value over the 64 lanes of a wave (every lane gets it):
// DPP row rotations, then the row and half swaps (as wave_sum_mod).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<0x121>(v));
    v = max(v, dpp_u32<0x122>(v));
    v = max(v, dpp_u32<0x124>(v));
    v = max(v, dpp_u32<0x128>(v));
    {
        uint32_t x = v, y = v;
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
        v = max(x, y);
    }
    {
        uint32_t x = v, y = v;
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
        v = max(x, y);
    }
    return v;
}

// Largest 64-bit key of a wave in two 32-bit passes: the high words, then the
// low words of the lanes whose high word is that maximum.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v)
{
    const uint32_t hi = (uint32_t)(v >> 32);
    const uint32_t mh = wave_max_u32(hi);
    const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)v : 0u);
    return join_u64(mh, ml);
}

// Top-k of keys held in registers by one wave: k rounds of a lane maximum and
// a wave maximum, the lane that holds the winner clearing it (keys are unique,
// so exactly one key is cleared per round; 0 means no candidate). Lane 0 writes
// the winners to dst[0..k) in rank order. NC keys per lane take part.
template <int NC>
__device__ __forceinline__ void wave_topk_n(uint64_t *key, int k, uint64_t *dst, int lane)
{
    for (int round = 0; round < k; ++round) {
        uint64_t best = key[0];
#pragma unroll
        for (int c = 1; c < NC; ++c) best = key[c] > best ? key[c] : best;
        const uint64_t win = wave_max_key(best);
#pragma unroll
        for (int c = 0; c < NC; ++c) key[c] = key[c] == win ? 0ull : key[c];
        if (lane == 0) dst[round] = win;
    }
}

// The same for the first nc (<= MAXC, wave-uniform) keys of each lane, the
// rest being 0: the rounds run over the next power of two of nc, so their cost
// follows the keys actually held.
template <int MAXC>
__device__ __forceinline__ void wave_topk(uint64_t (&key)[MAXC], int nc, int k, uint64_t *dst,
                                          int lane)
{
    nc = __builtin_amdgcn_readfirstlane(nc);
    if (nc <= 1)
        wave_topk_n<1>(key, k, dst, lane);
    else if (nc <= 2)
        wave_topk_n<(MAXC < 2 ? MAXC : 2)>(key, k, dst, lane);
    else if (nc <= 4)
        wave_topk_n<(MAXC < 4 ? MAXC : 4)>(key, k, dst, lane);
    else if (nc <= 8)
        wave_topk_n<(MAXC < 8 ? MAXC : 8)>(key, k, dst, lane);
    else
        wave_topk_n<MAXC>(key, k, dst, lane);
}

// Top-k of NL lists of k <= kRankMax keys each (list w at lists[w * STRIDE],
// in LDS) in one pass instead of k dependent rounds: every key is read by
// every lane (all reads issued before the first compare), lane i takes key
// (i / kRankMax, i % kRankMax) and counts the keys above it. Nonzero keys are
// unique (they embed the row), so they get the distinct ranks 0 .. nz - 1;
// the key of rank r < k goes to dst[r] and dst[nz .. k) gets 0 (no
// candidate), as wave_topk writes. Every slot has exactly one writer.
constexpr int kRankMax = 8;
template <int NL, int STRIDE>
__device__ __forceinline__ void wave_rank_merge(const uint64_t *lists, int k, uint64_t *dst,
                                                int lane)
{
    static_assert(NL * kRankMax <= 64, "one key per lane");
    uint64_t all[NL * kRankMax];
#pragma unroll
    for (int w = 0; w < NL; ++w)
#pragma unroll
        for (int r = 0; r < kRankMax; ++r) all[w * kRankMax + r] = r < k ? lists[w * STRIDE + r] : 0ull;
    const int lw = lane / kRankMax, lr = lane % kRankMax;
    const uint64_t mine = (lw < NL && lr < k) ? lists[lw * STRIDE + lr] : 0ull;
    int above[4] = {0, 0, 0, 0};   // four partial counts: shorter dependence chains
#pragma unroll
    for (int j = 0; j < NL * kRankMax; ++j) above[j & 3] += all[j] > mine ? 1 : 0;
    const int rank = (above[0] + above[1]) + (above[2] + above[3]);
    const int nz = __popcll(__ballot(mine != 0ull));
    if (mine != 0ull && rank < k) dst[rank] = mine;
    if (lane >= nz && lane < k) dst[lane] = 0ull;
}

// Workgroup-wide maximum of a key with one barrier: wave maxima go to
// scratch[wave], which the caller alternates between two buffers from one
// call to the next (a buffer is rewritten only after the next call's
// barrier, when every thread has read it).
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t *scratch)
{
    v = wave_max_u64(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nwaves = (blockDim.x + 63) >> 6;
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    uint64_t m = scratch[0];
    for (int w = 1; w < nwaves; ++w) m = scratch[w] > m ? scratch[w] : m;
    return m;
}

// Workgroup-wide sum over nwaves waves with one barrier (fixed order:
// deterministic).
template <int MAXW>
__device__ __forceinline__ float block_sum_f32(float v, float *scratch, int nwaves)
{
    v = wave_sum_mod<1>(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    float p[MAXW];   // every slot read at once, then added in wave order
#pragma unroll
    for (int w = 0; w < MAXW; ++w) p[w] = scratch[w];
    float r = p[0];
#pragma unroll
    for (int w = 1; w < MAXW; ++w)
        if (w < nwaves) r += p[w];
    return r;
}

// ----------------------------------------------------------- the kernel ---

// Persistent row-streaming kernel.
//  RPS  rows per sweep (threads t = u*RPS + r own unit u of row r of a sweep)
//  NMAT 1 (one matrix) or 2 (gate and up rows sharing the activation)
//  EPI  epilogue: store (3-way row split) / gated activation / logits + top-k
//  XS   how the activations are held (see XSrc)
//  D    sweeps whose loads are in flight while one sweep is computed
//  FMT  weight format (Q4_K, or Q6_K with f32 activations)
//  NG   wave groups: 1, or 2 for the gate/up pair, where the first half of the
//       workgroup streams the gate rows and the second half the same up rows
//       (each thread one matrix; twice the waves per compute unit, and the
//       busiest SIMD issues a quarter less arithmetic). Each row's partial sums
//       are formed by the same lanes and added in the same order either way.
// Workgroup w processes the contiguous sweeps from w*sq + min(w, srem), sq of
// them plus one for w < srem (or, interleaved, w, w+G, ...). The
// activation loads and the quant/header loads of the first D sweeps are
// issued first; then every step issues sweep i+D and computes sweep i. Wave
// partial sums go to an LDS bank; every fb sweeps one barrier publishes them
// and threads t < fb*RPS finish those rows.
template <int RPS, int NMAT, int EPI, int XS, int MAXT, int D, int FMT = FMT_Q4K, int NG = 1>
__global__ __launch_bounds__(MAXT) void rows_kernel(RowsArgs a)
{
    // Grid row y works on the y-th activation vector of a batch (one vector:
    // y = 0). The rows a workgroup streams depend only on blockIdx.x, so the
    // vectors after the first read the same rows, mostly from cache.
    args_to_sgprs(a);
    a.x += (int64_t)blockIdx.y * a.x_stride;
    a.o0 += (int64_t)blockIdx.y * a.o_stride;
    static_assert(RPS >= 1 && RPS <= 64 && (64 % RPS) == 0, "RPS must divide 64");
    static_assert(FMT == FMT_Q4K || (XS == XS_F32 && NMAT == 1),
                  "Q6_K: f32 activations, one matrix");
    static_assert(NG == 1 || (NG == 2 && NMAT == 2), "wave groups split a matrix pair");
    // matrices one thread streams
    constexpr int LM = NG == 2 ? 1 : NMAT;
    constexpr int NW = MAXT / 64;
    constexpr int FB = EPI == EPI_LOGITS ? Q4K_LMHEAD_FB : Q4K_ROWS_FB;
    constexpr bool kInt = XS != XS_F32;
    __shared__ float red[2][NW][FB * NMAT * RPS];
    __shared__ float lg[EPI == EPI_LOGITS ? kLmheadRowsPerWgMax : 1];
    __shared__ uint64_t wave_lists[EPI == EPI_LOGITS ? NW : 1][EPI == EPI_LOGITS ? kTopkMax : 1];
    __shared__ float sum_scratch[EPI == EPI_LOGITS ? NW : 1];
    __shared__ uint64_t max_scratch[EPI == EPI_LOGITS ? NW : 1];
    __shared__ float base_scratch[EPI == EPI_LOGITS ? NW : 1];
    __shared__ float norm_scratch[NW];
    extern __shared__ uint4 xlds_v[];   // XS_LDS: planes of x (planes_bytes(cols))
    uint8_t *const xlds = reinterpret_cast<uint8_t *>(xlds_v);

    const int t = threadIdx.x;
    const int nthr = a.nthr;   // blockDim.x
    const int wave = t >> 6, lane = t & 63;
    const int nwaves = nthr >> 6;
    // wave group of the thread (uniform across a wave: the group size is a
    // multiple of 64), its thread and wave index inside the group
    const int gsz = nthr / NG;
    static_assert(NG == 1 || NG == 2, "one or two wave groups");
    const int grp = NG == 1 ? 0 : __builtin_amdgcn_readfirstlane(t >= gsz ? 1 : 0);
    const int tl = t - grp * gsz;
    const int gwave = tl >> 6;
    // sweeps per reduction batch: every row of a batch needs a thread
    const int fb = min(FB, (nthr / RPS));
    const int u = tl / RPS;
    const int r = tl % RPS;
    const bool uact = u < a.U;
    const int b = u >> 2, g = u & 3;
    const int sh = (g & 1) * 16;
    const bool upper = g >= 2;
    const int64_t cols = (int64_t)a.nb * kQK;
    const int64_t rowbytes = (int64_t)a.nb * fmt_block_bytes(FMT);
    const int64_t unit_off = (int64_t)b * fmt_block_bytes(FMT);
    // The workgroup's sweeps, by local index i = 0 .. n_loc-1: either the
    // contiguous range [s_begin, s_end), or (ilv) sweeps w, w+G, w+2G, ... so
    // that all workgroups move through the matrix together.
    const bool ilv = a.ilv != 0;
    // (The split comes from the host: a 64-bit division here costs hundreds
    // of instructions ahead of the first load.)
    const int64_t G = a.nwg, wg = blockIdx.x;
    const int64_t n_loc = a.sq + (wg < a.srem ? 1 : 0);
    const int64_t s_begin = ilv ? wg : wg * a.sq + (wg < a.srem ? wg : (int64_t)a.srem);
    const int64_t s_step = ilv ? G : 1;
    auto gsweep = [&](int64_t i) -> int64_t { return s_begin + i * s_step; };
    // first row the resource starts at; rows of this workgroup: [row_begin, row_span_end)
    const int64_t row_begin = ilv ? 0 : s_begin * RPS;
    const int64_t row_span_end = ilv ? a.rows : min((s_begin + n_loc) * RPS, a.rows);

    // Buffer resources over this workgroup's rows (the host keeps the span
    // below 2^30 bytes); offsets are relative to row_begin. Q6_K rows start at
    // even bytes only: the resource then begins at the 4-byte boundary below
    // (lead bytes of the previous row, never read as part of this one).
    __amdgpu_buffer_rsrc_t rs[LM];
    uint32_t lead = 0;
#pragma unroll
    for (int m = 0; m < LM; ++m) {
        const uint8_t *base = ((m + grp) == 0 ? a.W0 : a.W1) + row_begin * rowbytes;
        if (FMT == FMT_Q6K) lead = (uint32_t)((uintptr_t)base & 3u);
        rs[m] = make_rsrc(base - lead, (uint32_t)((row_span_end - row_begin) * rowbytes) + lead);
    }
    const uint32_t qoff = 16u + 32u * (uint32_t)g;
    auto slot_off = [&](int64_t i) -> uint32_t {
        const int64_t row = gsweep(i) * RPS + r;
        return (uact && i < n_loc && row < a.rows)
                   ? (uint32_t)((row - row_begin) * rowbytes + unit_off) + lead
                   : kOutOfRange;
    };

    // ---- activation loads go out first, then the first D sweeps ----
    // XS_LDS: this thread's first groups of 8 activations (the conversion
    // passes loaded up front); XS_THREAD / XS_F32: the unit's 64 floats.
    // With a fused norm, its inputs for the first group (XS_LDS) or the first
    // two steps of the norm pass (XS_F32 staging through LDS) go out here too.
    const int ngroups = (int)(cols / 8);
    const int n4 = (int)(cols / 4);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(cols * 4));
    const bool norm = a.nw != nullptr;
    const bool z_lds = norm && XS == XS_F32 && FMT == FMT_Q4K && cols <= kNormLdsCols;
    const __amdgpu_buffer_rsrc_t rdel = make_rsrc(a.delta, a.delta ? (uint32_t)(cols * 4) : 0u);
    const __amdgpu_buffer_rsrc_t rnw = make_rsrc(a.nw, norm ? (uint32_t)(cols * 4) : 0u);
    // XS_LDS without a norm: the activations of the first kXPre conversion
    // passes are all loaded up front (one memory latency instead of one per
    // pass; rows of 2048 or more columns at RPS <= 2 take several passes).
    constexpr int kWlPasses = (512 / RPS + 63) / 64;
    constexpr int kXPre = kWlPasses < 4 ? kWlPasses : 4;
    uint4 xv[XS == XS_LDS ? 2 * kXPre : 16];
    uint32_t xoff[XS == XS_LDS ? 1 : 16];
    uint4 nv[XS == XS_LDS ? 4 : 6];   // norm inputs issued with x (see above)
    // XS_LDS group mapping. Without a norm (no row-wide sum of squares), each
    // wave converts exactly the gpw = 512/RPS groups of 8 activations its own
    // units read (units 64w/RPS .. 64(w+1)/RPS - 1), lane l taking groups
    // gbase + l + 64i, so no workgroup barrier is needed before the planes are
    // read: LDS accesses of one wave complete in order. With a norm, thread t
    // takes groups t, t + blockDim, ... and a barrier publishes the planes.
    const bool wave_local = Q4K_WAVE_LOCAL_X && XS == XS_LDS && a.nw == nullptr;
    const int gpw = 512 / RPS;
    const int gbase = gwave * gpw;
    // activation planes in LDS: one copy per wave group when each wave converts
    // its own (no barrier between the groups), else one shared copy
    uint8_t *const xp = xlds + (wave_local ? (int64_t)grp * planes_bytes(cols) : 0);
    const int gpasses = wave_local ? (gpw + 63) / 64 : a.xpass;
    // group of pass i of this thread, or ngroups for none
    auto group_of = [&](int i) -> int {
        if (wave_local) {
            const int l = lane + 64 * i;
            return (l < gpw && gbase + l < ngroups) ? gbase + l : ngroups;
        }
        const int e = t + i * nthr;
        return e < ngroups ? e : ngroups;
    };
    if (XS == XS_LDS) {
        const int e0 = group_of(0);
        const uint32_t xo = e0 < ngroups ? (uint32_t)e0 * 32u : kOutOfRange;
        xv[0] = bload16(rx, xo);
        xv[1] = bload16(rx, xo + 16u);
        if (norm) {
            nv[0] = bload16(rdel, xo);
            nv[1] = bload16(rdel, xo + 16u);
            nv[2] = bload16(rnw, xo);
            nv[3] = bload16(rnw, xo + 16u);
        } else {
#pragma unroll
            for (int i = 1; i < kXPre; ++i) {
                const int e = group_of(i);
                const uint32_t xoi = (wave_local && e < ngroups) ? (uint32_t)e * 32u : kOutOfRange;
                xv[2 * i] = bload16(rx, xoi);
                xv[2 * i + 1] = bload16(rx, xoi + 16u);
            }
        }
    } else {
        if (FMT == FMT_Q6K) {
            // quarters j = 0..3 of unit (b, n, h): x[256b + 128n + 32j + 16h + i]
            const uint32_t xo =
                uact ? (uint32_t)(256 * b + 128 * (g >> 1) + 16 * (g & 1)) * 4u : kOutOfRange;
#pragma unroll
            for (int i = 0; i < 16; ++i) xoff[i] = xo + 128u * (i / 4) + 16u * (i % 4);
        } else {
            const uint32_t xo = uact ? (uint32_t)(64 * u) * 4u : kOutOfRange;
#pragma unroll
            for (int i = 0; i < 16; ++i) xoff[i] = xo + 16u * i;
        }
        if (z_lds) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int i = t + k * nthr;
                const uint32_t off = i < n4 ? (uint32_t)i * 16u : kOutOfRange;
                nv[3 * k] = bload16(rx, off);
                nv[3 * k + 1] = bload16(rdel, off);
                nv[3 * k + 2] = bload16(rnw, off);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) xv[i] = bload16(rx, xoff[i]);
        }
    }
    // The activation loads must leave before the weight loads: the wait
    // counter is in order, so waiting for x would otherwise also wait for the
    // first sweeps of weights. A compiler barrier keeps that order.
    asm volatile("" ::: "memory");

    using SlotT = std::conditional_t<FMT == FMT_Q6K, Slot6<LM>, Slot<LM>>;
    auto issue = [&](SlotT &sl, uint32_t off) {
        if constexpr (FMT == FMT_Q6K)
            load_slot6<LM>(sl, rs, off, g >> 1, g & 1);
        else
            load_slot<LM>(sl, rs, off, qoff);
    };
    // The first kPre sweeps go out before the activations are prepared, the
    // rest of the first D right after (a deeper early burst delays the
    // activation reads, which every sweep waits for).
    constexpr int kPre = D < Q4K_PRE_SWEEPS ? D : Q4K_PRE_SWEEPS;
    SlotT buf[D + 1];
#pragma unroll
    for (int j = 0; j < kPre; ++j) issue(buf[j], slot_off(j));

    // ---- fused RMSNorm ----
    // s = x + delta (f32) over the whole row (every workgroup reads it from L2),
    // its sum of squares, and the new residual stream (workgroup 0). With
    // activations converted in LDS this rides on the conversion loop below;
    // otherwise one cooperative pass does it here and, for rows that fit,
    // also leaves z = s * nw in LDS, so that the thread's own 64 activations
    // are read from there: one memory round trip either way.
    float *const zl = reinterpret_cast<float *>(xlds);
    float inv_rms = 1.f;
    float ss_part = 0.f;
    float4 *const o4 = (norm && blockIdx.x == 0) ? reinterpret_cast<float4 *>(a.h_out) : nullptr;
    // s of four activations (x, delta and nw given), and z = s * nw
    auto norm4 = [&](uint4 hv, uint4 dv, uint4 wv, float4 &sv) -> uint4 {
        sv = make_float4(__uint_as_float(hv.x), __uint_as_float(hv.y), __uint_as_float(hv.z),
                         __uint_as_float(hv.w));
        if (a.delta) {
            sv.x += __uint_as_float(dv.x); sv.y += __uint_as_float(dv.y);
            sv.z += __uint_as_float(dv.z); sv.w += __uint_as_float(dv.w);
        }
        return make_uint4(__float_as_uint(sv.x * __uint_as_float(wv.x)),
                          __float_as_uint(sv.y * __uint_as_float(wv.y)),
                          __float_as_uint(sv.z * __uint_as_float(wv.z)),
                          __float_as_uint(sv.w * __uint_as_float(wv.w)));
    };
    auto add_sq = [&](const float4 &v) {
        ss_part = fmaf(v.x, v.x, ss_part);
        ss_part = fmaf(v.y, v.y, ss_part);
        ss_part = fmaf(v.z, v.z, ss_part);
        ss_part = fmaf(v.w, v.w, ss_part);
    };
    if constexpr (XS != XS_LDS) if (norm) {
        auto pass_step = [&](int i, uint4 hv, uint4 dv, uint4 wv) {
            float4 sv;
            const uint4 z = norm4(hv, dv, wv, sv);
            add_sq(sv);
            if (o4) o4[i] = sv;
            if (z_lds) reinterpret_cast<uint4 *>(zl)[xslot(i)] = z;
        };
        int i0 = t;
        if (z_lds) {   // the first two steps were loaded with x
            if (t < n4) pass_step(t, nv[0], nv[1], nv[2]);
            if (t + nthr < n4) pass_step(t + nthr, nv[3], nv[4], nv[5]);
            i0 = t + 2 * nthr;
        }
        for (int i = i0; i < n4; i += nthr) {
            const uint32_t off = (uint32_t)i * 16u;
            pass_step(i, bload16(rx, off), bload16(rdel, off), bload16(rnw, off));
        }
        const float ss = block_sum_f32<NW>(ss_part, norm_scratch, nwaves);   // also publishes zl
        inv_rms = 1.f / sqrtf(ss / (float)cols + a.eps);
    }

    // ---- the thread's activations (unused units: zeros) ----
    XUnit xu;
    XF32 xf;
    // block-floating-point launches: this wave covers a sub-block beyond the
    // spread and computes with f32 activations (wave-uniform)
    bool wave_f32 = false;
    float s6[4] = {0.f, 0.f, 0.f, 0.f};   // Q6_K: sums of the four quarters
    if (XS == XS_THREAD || XS == XS_F32) {
        if (z_lds) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                xv[i] = uact ? reinterpret_cast<const uint4 *>(xlds)[17 * u + i]
                             : make_uint4(0, 0, 0, 0);
        } else if (norm) {
            float4 sv;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                xv[i] = norm4(xv[i], bload16(rdel, xoff[i]), bload16(rnw, xoff[i]), sv);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xf.xa[4 * i + 0] = __uint_as_float(xv[i].x); xf.xa[4 * i + 1] = __uint_as_float(xv[i].y);
            xf.xa[4 * i + 2] = __uint_as_float(xv[i].z); xf.xa[4 * i + 3] = __uint_as_float(xv[i].w);
            xf.xb[4 * i + 0] = __uint_as_float(xv[8 + i].x); xf.xb[4 * i + 1] = __uint_as_float(xv[8 + i].y);
            xf.xb[4 * i + 2] = __uint_as_float(xv[8 + i].z); xf.xb[4 * i + 3] = __uint_as_float(xv[8 + i].w);
        }
        if (XS == XS_THREAD) {
            float pA[24], pB[24], XA, XB, SA, SB;
            const bool okA = planes32(xf.xa, pA, XA, SA);
            const bool okB = planes32(xf.xb, pB, XB, SB);
            wave_f32 = __builtin_amdgcn_ballot_w64(uact && !(okA && okB)) != 0;
            if (wave_f32) {
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    xu.r[i] = xf.xa[i];
                    xu.r[32 + i] = xf.xb[i];
                }
                xu.r[64] = SA;
                xu.r[65] = SB;
            } else {
#pragma unroll
                for (int i = 0; i < 24; ++i) {
                    xu.r[i] = pA[i];
                    xu.r[24 + i] = pB[i];
                }
                xu.r[48] = XA;
                xu.r[49] = XB;
                xu.r[50] = SA;
                xu.r[51] = SB;
            }
        } else {
            xf.SA = xf.SB = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                xf.SA += xf.xa[i];
                xf.SB += xf.xb[i];
            }
            if (FMT == FMT_Q6K) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float *xj = j < 2 ? &xf.xa[16 * j] : &xf.xb[16 * (j - 2)];
                    s6[j] = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) s6[j] += xj[i];
                }
            }
        }
    } else {
        // Cooperative conversion: 4 threads per 32-activation sub-block, 8
        // activations each; max and sum over the 4 lanes of a quad (DPP).
        float *Xs = reinterpret_cast<float *>(xp + 3 * cols);
        float *Ss = Xs + cols / 32;
        // group e of 8 activations (x, and with a norm delta and nw, given)
        auto convert = [&](int e, uint4 h0, uint4 h1, uint4 d0, uint4 d1, uint4 w0, uint4 w1) {
            if (norm) {
                float4 s0, s1;
                h0 = norm4(h0, d0, w0, s0);
                h1 = norm4(h1, d1, w1, s1);
                add_sq(s0);
                add_sq(s1);
                if (o4 && e < ngroups) {
                    o4[2 * e] = s0;
                    o4[2 * e + 1] = s1;
                }
            }
            const float v[8] = {__uint_as_float(h0.x), __uint_as_float(h0.y),
                                __uint_as_float(h0.z), __uint_as_float(h0.w),
                                __uint_as_float(h1.x), __uint_as_float(h1.y),
                                __uint_as_float(h1.z), __uint_as_float(h1.w)};
            float amax = 0.f, sum = 0.f, abssum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                amax = fmaxf(amax, fabsf(v[i]));
                sum += v[i];
                abssum += fabsf(v[i]);
            }
#if Q4K_DPP_QUAD
            // quad_perm [1,0,3,2] and [2,3,0,1]: lane ^ 1, lane ^ 2
            amax = fmaxf(amax, dpp_f32<0xB1>(amax));
            sum += dpp_f32<0xB1>(sum);
            abssum += dpp_f32<0xB1>(abssum);
            amax = fmaxf(amax, dpp_f32<0x4E>(amax));
            sum += dpp_f32<0x4E>(sum);
            abssum += dpp_f32<0x4E>(abssum);
#else
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            sum += __shfl_xor(sum, 1);
            abssum += __shfl_xor(abssum, 1);
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            sum += __shfl_xor(sum, 2);
            abssum += __shfl_xor(abssum, 2);
#endif
            int shift;
            float X;
            bfp_params(amax, sum, shift, X);
            // a negative scale marks a sub-block beyond the spread
            if (!bfp_spread_ok(amax, abssum)) X = -1.0f;
            uint32_t p[3][2];
            pack4((uint32_t)to_int22(v[0], shift), (uint32_t)to_int22(v[1], shift),
                  (uint32_t)to_int22(v[2], shift), (uint32_t)to_int22(v[3], shift), p[0][0],
                  p[1][0], p[2][0]);
            pack4((uint32_t)to_int22(v[4], shift), (uint32_t)to_int22(v[5], shift),
                  (uint32_t)to_int22(v[6], shift), (uint32_t)to_int22(v[7], shift), p[0][1],
                  p[1][1], p[2][1]);
            if (e < ngroups) {
#pragma unroll
                for (int pl = 0; pl < 3; ++pl)
                    *reinterpret_cast<uint2 *>(xp + pl * cols + 8 * e) =
                        make_uint2(p[pl][0], p[pl][1]);
                if ((e & 3) == 0) {
                    Xs[e >> 2] = X;
                    Ss[e >> 2] = sum;
                }
            }
        };
        // The first group was loaded before the weights; later ones (rows
        // wider than 8 * blockDim) are loaded here. Trip counts are uniform
        // (blockDim % 4 == 0), so the xor shuffles see whole quads.
        const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
        convert(group_of(0), xv[0], xv[1], norm ? nv[0] : zero4, norm ? nv[1] : zero4,
                norm ? nv[2] : zero4, norm ? nv[3] : zero4);
        if (wave_local) {
#pragma unroll
            for (int i = 1; i < kXPre; ++i)
                convert(group_of(i), xv[2 * i], xv[2 * i + 1], zero4, zero4, zero4, zero4);
        }
        for (int i = wave_local ? kXPre : 1; i < gpasses; ++i) {
            const int e = group_of(i);
            const uint32_t xo = e < ngroups ? (uint32_t)e * 32u : kOutOfRange;
            const uint4 h0 = bload16(rx, xo), h1 = bload16(rx, xo + 16u);
            uint4 d0 = zero4, d1 = zero4, w0 = zero4, w1 = zero4;
            if (norm) {
                d0 = bload16(rdel, xo);
                d1 = bload16(rdel, xo + 16u);
                w0 = bload16(rnw, xo);
                w1 = bload16(rnw, xo + 16u);
            }
            convert(e, h0, h1, d0, d1, w0, w1);
        }
        if (norm) {
            const float ss = block_sum_f32<NW>(ss_part, norm_scratch, nwaves);   // also publishes the planes
            inv_rms = 1.f / sqrtf(ss / (float)cols + a.eps);
        } else if (wave_local) {
            // the wave reads back only what it wrote: keep the compiler from
            // moving the reads above the writes
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        } else {
            __syncthreads();
        }
        // This unit's planes: 64 bytes per plane at 64u, X and S at 2u.
        if (uact) {
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) {
                const uint4 *q = reinterpret_cast<const uint4 *>(xp + pl * cols + 64 * u);
                const uint4 qv[4] = {q[0], q[1], q[2], q[3]};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    float *dst = xu.r + (h < 2 ? 0 : 24) + 8 * pl + 4 * (h & 1);
                    dst[0] = __uint_as_float(qv[h].x);
                    dst[1] = __uint_as_float(qv[h].y);
                    dst[2] = __uint_as_float(qv[h].z);
                    dst[3] = __uint_as_float(qv[h].w);
                }
            }
            xu.r[48] = Xs[2 * u];
            xu.r[49] = Xs[2 * u + 1];
            xu.r[50] = Ss[2 * u];
            xu.r[51] = Ss[2 * u + 1];
        } else {
#pragma unroll
            for (int i = 0; i < 52; ++i) xu.r[i] = 0.f;
        }
        wave_f32 = __builtin_amdgcn_ballot_w64(uact && (xu.r[48] < 0.f || xu.r[49] < 0.f)) != 0;
        if (wave_f32) {
            // f32 activations of this unit, read again (with a fused norm,
            // s * w recomputed from its inputs; the 1/rms scale is applied to
            // the outputs as on the block-floating-point path)
            const uint32_t xo = uact ? (uint32_t)(64 * u) * 4u : kOutOfRange;
            uint4 fv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) fv[i] = bload16(rx, xo + 16u * i);
            if (norm) {
                float4 sv;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    fv[i] = norm4(fv[i], bload16(rdel, xo + 16u * i), bload16(rnw, xo + 16u * i), sv);
            }
            float SA = 0.f, SB = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float *dst = xu.r + 4 * i;
                dst[0] = __uint_as_float(fv[i].x);
                dst[1] = __uint_as_float(fv[i].y);
                dst[2] = __uint_as_float(fv[i].z);
                dst[3] = __uint_as_float(fv[i].w);
            }
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                SA += xu.r[i];
                SB += xu.r[32 + i];
            }
            xu.r[64] = SA;
            xu.r[65] = SB;
        }
    }

    // One sweep: dot products, wave reduction, and every fb sweeps the
    // cross-wave reduction and epilogue of that batch of rows.
#pragma unroll
    for (int j = kPre; j < D; ++j) issue(buf[j], slot_off(j));

    int kb = 0, bank = 0;
    auto compute_sweep = [&](const SlotT &sl, int64_t sj) {
#pragma unroll
        for (int m = 0; m < LM; ++m) {
            float v;
            if constexpr (FMT == FMT_Q6K)
                v = unit_dot_q6(sl.q[m], sl.sc[m], sl.d[m], sl.mis, xf, s6, g & 1);
            else if constexpr (!kInt)
                v = unit_dot_f32(sl.q[m], sl.h[m], xf, sh, upper);
            else  // wave-uniform choice: f32 activations for a wave beyond the spread
                v = wave_f32 ? unit_dot_f32u(sl.q[m], sl.h[m], xu, sh, upper)
                             : unit_dot(sl.q[m], sl.h[m], xu, sh, upper);
            v = wave_sum_mod<RPS>(v);
            if (lane < RPS) red[bank][wave][(kb * NMAT + m + grp) * RPS + lane] = v;
        }
        ++kb;
        if (kb == fb || sj == n_loc - 1) {
            __syncthreads();
            if (t < kb * RPS) {
                const int k = t / RPS, rr = t % RPS;
                const int64_t li = sj - kb + 1 + k;         // local sweep of this row
                const int64_t row = gsweep(li) * RPS + rr;
                if (row < a.rows) {
                    // Wave partials added in wave order. Every slot a launch
                    // of this shape can hold is read first (all reads in
                    // flight together), and only the waves present are added.
                    float v0 = 0.f, v1 = 0.f;
                    if (NG == 1) {
                        float p0[NW], p1[NW];
#pragma unroll
                        for (int w = 0; w < NW; ++w) {
                            p0[w] = red[bank][w][(k * NMAT + 0) * RPS + rr];
                            p1[w] = NMAT == 2 ? red[bank][w][(k * NMAT + 1) * RPS + rr] : 0.f;
                        }
#pragma unroll
                        for (int w = 0; w < NW; ++w) {
                            if (w < nwaves) {
                                v0 += p0[w];
                                if (NMAT == 2) v1 += p1[w];
                            }
                        }
                    } else {
                        // gate partials from the first group's waves, up from the second's
                        const int gw = nwaves / 2;
                        float p0[NW / 2], p1[NW / 2];
#pragma unroll
                        for (int w = 0; w < NW / 2; ++w) {
                            p0[w] = red[bank][w][(k * NMAT + 0) * RPS + rr];
                            p1[w] = red[bank][gw + w][(k * NMAT + 1) * RPS + rr];
                        }
#pragma unroll
                        for (int w = 0; w < NW / 2; ++w) {
                            if (w < gw) {
                                v0 += p0[w];
                                v1 += p1[w];
                            }
                        }
                    }
                    if (norm) {
                        v0 *= inv_rms;
                        v1 *= inv_rms;
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
                        lg[li * RPS + rr] = v0;
                    }
                }
            }
            kb = 0;
            bank ^= 1;
        }
    };

    // Full groups of D+1 sweeps: step j issues sweep s+j+D into the slot freed
    // by step j-1 and computes sweep s+j. No early exit inside a group keeps
    // the ring's wait counts exact (only the oldest sweep is waited for).
    // Prefetches past the workgroup's last sweep read zeros.
    int64_t s = 0;
    for (; s + D < n_loc; s += D + 1) {
#pragma unroll
        for (int j = 0; j <= D; ++j) {
            if (D > 0) issue(buf[(j + D) % (D + 1)], slot_off(s + j + D));
            if (D == 0) issue(buf[0], slot_off(s + j));
            compute_sweep(buf[j], s + j);
        }
    }
    // Tail: fewer than D+1 sweeps left, all already in flight in buf[0..].
#pragma unroll
    for (int j = 0; j < (D > 0 ? D : 1); ++j) {
        if (s + j < n_loc) {
            if (D == 0) issue(buf[0], slot_off(s + j));
            compute_sweep(buf[j], s + j);
        }
    }

    if (EPI == EPI_LOGITS) {
        // Per-workgroup top-k of its rows, written in rank order, and (with
        // stats) the workgroup's softmax partial, computed side by side: four
        // waves (one per SIMD) each take the top-k of a quarter of the rows,
        // held as orderable keys in registers (k rounds of a lane maximum and
        // a wave maximum, the lane holding the winner clearing it; keys are
        // unique: they embed the row), while each other wave forms the partial
        // of its share of the rows. Wave 0 then merges the four lists the same
        // way, and the partials are combined beside it.
        __syncthreads();
        // local row j = i * RPS + rr is global row gsweep(i) * RPS + rr; rows
        // past the end (a partial last sweep) are skipped
        const int n = (int)(n_loc * RPS);
        auto grow = [&](int j) -> int64_t { return gsweep(j / RPS) * RPS + j % RPS; };
        uint64_t *out = a.cand + (int64_t)blockIdx.x * a.k;
        constexpr int kTkWaves = 4;   // every launch has at least four waves
        // quarters of at most kLmheadRowsPerWgMax / 4 rows
        constexpr int kKeysPerLane = kLmheadRowsPerWgMax / (kTkWaves * 64);
        const bool stats = a.stats != nullptr;
        const int swaves = nwaves - kTkWaves;   // waves that sum the exponentials
        // Softmax partial of the workgroup: m = its largest logit (its first
        // winner: the largest key, NaN lowest), s = sum of exp(l - m). When m
        // is -inf (every row -inf or NaN) the exponent is taken against 0
        // instead, so that -inf rows add 0 and NaN rows poison the sum. A
        // share of the rows gives (m_w, s_w) the same way (base b_w), and the
        // shares combine as s = sum over s_w != 0 of s_w exp(b_w - b): b_w <= b,
        // so no term overflows, and a NaN s_w still poisons the sum.
        auto share_partial = [&](int j0, int step, uint64_t &mk, float &bw, float &sw) {
            mk = 0;
            for (int j = j0; j < n; j += step) {
                const int64_t gr = grow(j);
                if (gr < a.rows) {
                    const uint64_t kk = topk_key(lg[j], (uint32_t)gr);
                    mk = kk > mk ? kk : mk;
                }
            }
            mk = wave_max_u64(mk);
            const float mw = topk_key_value(mk);
            bw = mw == -INFINITY ? 0.f : mw;
            sw = 0.f;
            for (int j = j0; j < n; j += step)
                if (grow(j) < a.rows) sw += expf(lg[j] - bw);
            sw = wave_sum_mod<1>(sw);
        };
        if (wave < kTkWaves) {
            const int per_wave = (n + kTkWaves - 1) / kTkWaves;
            const int cpl = (per_wave + 63) / 64;
            uint64_t key[kKeysPerLane];
#pragma unroll
            for (int c = 0; c < kKeysPerLane; ++c) {
                const int o = c * 64 + lane;
                const int j = wave * per_wave + o;
                uint64_t kk = 0;
                if (c < cpl && o < per_wave && j < n) {
                    const int64_t gr = grow(j);
                    if (gr < a.rows) kk = topk_key(lg[j], (uint32_t)gr);
                }
                key[c] = kk;
            }
            wave_topk(key, cpl, a.k, wave_lists[wave], lane);
        }
        // the waves beyond the four take the partial; four-wave launches take it
        // after their lists (every wave a quarter of the rows)
        if (stats && (wave >= kTkWaves || swaves == 0)) {
            const int sw_idx = swaves > 0 ? wave - kTkWaves : wave;
            const int sw_n = swaves > 0 ? swaves : nwaves;
            uint64_t mk;
            float bw, sw;
            share_partial(lane + 64 * sw_idx, 64 * sw_n, mk, bw, sw);
            if (lane == 0) {
                max_scratch[sw_idx] = mk;
                base_scratch[sw_idx] = bw;
                sum_scratch[sw_idx] = sw;
            }
        }
        __syncthreads();
        if (wave == 0) {
            if (a.k <= kRankMax) {
                wave_rank_merge<kTkWaves, kTopkMax>(&wave_lists[0][0], a.k, out, lane);
            } else {
                constexpr int kMergePerLane = kTkWaves * kTopkMax / 64;
                const int total = kTkWaves * a.k;
                const int mpl = (total + 63) / 64;
                uint64_t m[kMergePerLane];
#pragma unroll
                for (int c = 0; c < kMergePerLane; ++c) {
                    const int i = c * 64 + lane;
                    m[c] = (c < mpl && i < total) ? wave_lists[i / a.k][i % a.k] : 0ull;
                }
                wave_topk(m, mpl, a.k, out, lane);
            }
        } else if (stats && t == 64) {   // beside wave 0's merge
            // all of the shares' partials read at once, then combined in order
            const int nsum = swaves > 0 ? swaves : nwaves;
            uint64_t pm[NW];
            float pb[NW], ps[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                pm[w] = max_scratch[w];
                pb[w] = base_scratch[w];
                ps[w] = sum_scratch[w];
            }
            uint64_t mk = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if (w < nsum) mk = pm[w] > mk ? pm[w] : mk;
            const float wg_max = topk_key_value(mk);
            const float base = wg_max == -INFINITY ? 0.f : wg_max;
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if (w < nsum && ps[w] != 0.f) sum += ps[w] * expf(pb[w] - base);
            a.stats[blockIdx.x] = make_float2(wg_max, sum);
        }
    }
}

// Merge of the per-workgroup candidate lists (each sorted in rank order) into
// the global top-k. Fast path (all candidates fit kMergeRegKeys per thread):
// every key is loaded into registers with all loads in flight, each wave takes
// the top-k of its share (wave_topk: no barriers) and wave 0 the top-k of the
// four waves' lists. Otherwise a k-way merge: thread t owns lists t, t+256,
// ...; each round the workgroup takes the largest list head and that list
// advances (lists staged in LDS when they fit).
// With stats, the per-workgroup softmax partials (m_w, s_w) are combined
// against M, the largest logit (the first winner): S = sum_w s_w exp(m_w - M),
// lse = M + log S, and a winner's probability is exp(l - M) / S.
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeListsPerThread = 4;   // up to 1024 lists
constexpr int kMergeStagedPerThread = 24; // 48 KB of staged candidates
constexpr int kMergeLdsKeys = kMergeStagedPerThread * kMergeThreads;
constexpr int kMergeRegKeys = 16;         // fast path: candidate keys per thread

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(const uint64_t *cand, int nlists,
                                                                    int k, const float *logits,
                                                                    int32_t *top_idx,
                                                                    float *top_val,
                                                                    const float2 *stats,
                                                                    float *top_prob, float *lse)
{
    __shared__ uint64_t key_scratch[2][kMergeWaves];
    __shared__ float sum_scratch[kMergeWaves];
    __shared__ uint64_t staged[kMergeLdsKeys];
    __shared__ uint64_t wave_wins[kMergeWaves][kTopkMax];
    __shared__ uint64_t wins[kTopkMax];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int total = nlists * k;
    // the partials and the candidates are loaded together: one memory latency
    float2 st[kMergeListsPerThread];
#pragma unroll
    for (int i = 0; i < kMergeListsPerThread; ++i) {
        const int l = t + i * kMergeThreads;
        st[i] = (stats && l < nlists) ? stats[l] : make_float2(-INFINITY, 0.f);
    }
    if (total <= kMergeThreads * kMergeRegKeys) {
        const int per_wave = (total + kMergeWaves - 1) / kMergeWaves;
        const int cpl = (per_wave + 63) / 64;
        uint64_t key[kMergeRegKeys];
#pragma unroll
        for (int c = 0; c < kMergeRegKeys; ++c) {
            const int o = c * 64 + lane;
            const int i = wave * per_wave + o;
            key[c] = (c < cpl && o < per_wave && i < total) ? cand[i] : 0ull;
        }
        wave_topk(key, cpl, k, wave_wins[wave], lane);
        __syncthreads();
        if (wave == 0) {
            if (k <= kRankMax) {
                wave_rank_merge<kMergeWaves, kTopkMax>(&wave_wins[0][0], k, wins, lane);
            } else {
                constexpr int kPer = kMergeWaves * kTopkMax / 64;
                const int tot2 = kMergeWaves * k;
                const int mpl = (tot2 + 63) / 64;
                uint64_t m[kPer];
#pragma unroll
                for (int c = 0; c < kPer; ++c) {
                    const int i = c * 64 + lane;
                    m[c] = (c < mpl && i < tot2) ? wave_wins[i / k][i % k] : 0ull;
                }
                wave_topk(m, mpl, k, wins, lane);
            }
        }
    } else {
        const bool in_lds = total <= kMergeLdsKeys;
        if (in_lds) {
            uint64_t v[kMergeStagedPerThread];
#pragma unroll
            for (int i = 0; i < kMergeStagedPerThread; ++i) {
                const int j = t + i * kMergeThreads;
                v[i] = j < total ? cand[j] : 0ull;
            }
#pragma unroll
            for (int i = 0; i < kMergeStagedPerThread; ++i) {
                const int j = t + i * kMergeThreads;
                if (j < total) staged[j] = v[i];
            }
        }
        __syncthreads();
        auto key_at = [&](int l, int pos) -> uint64_t {
            const int i = l * k + pos;
            return in_lds ? staged[i] : cand[i];
        };
        int pos[kMergeListsPerThread];
        uint64_t head[kMergeListsPerThread];
#pragma unroll
        for (int i = 0; i < kMergeListsPerThread; ++i) {
            const int l = t + i * kMergeThreads;
            pos[i] = 0;
            head[i] = l < nlists ? key_at(l, 0) : 0ull;
        }
        for (int round = 0; round < k; ++round) {
            uint64_t best = 0;
#pragma unroll
            for (int i = 0; i < kMergeListsPerThread; ++i) best = head[i] > best ? head[i] : best;
            const uint64_t win = block_max_u64(best, key_scratch[round & 1]);
            if (win != 0) {
#pragma unroll
                for (int i = 0; i < kMergeListsPerThread; ++i) {
                    if (head[i] == win) {  // keys are unique (they embed the row)
                        const int l = t + i * kMergeThreads;
                        ++pos[i];
                        head[i] = pos[i] < k ? key_at(l, pos[i]) : 0ull;
                    }
                }
            }
            if (t == 0) wins[round] = win;
        }
    }
    __syncthreads();   // publishes wins[]
    const float M = topk_key_value(wins[0]);
    const float base = M == -INFINITY ? 0.f : M;
    float S = 0.f;
    if (stats) {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < kMergeListsPerThread; ++i)
            if (st[i].y != 0.f) sum += st[i].y * expf(st[i].x - base);  // NaN partials propagate
        S = block_sum_f32<kMergeWaves>(sum, sum_scratch, kMergeWaves);
    }
    if (t < k) {
        const uint64_t win = wins[t];
        if (win == 0) {
            top_idx[t] = -1;
            top_val[t] = __uint_as_float(0x7FC00000u);
            if (stats) top_prob[t] = __uint_as_float(0x7FC00000u);
        } else {
            const uint32_t idx = ~(uint32_t)(win & 0xFFFFFFFFu);
            // the key holds the logit's bits, except the sign of a zero and a
            // NaN's payload: only those are read back from the logits
            float l = topk_key_value(win);
            if (!(fabsf(l) > 0.f)) l = logits[idx];
            top_idx[t] = (int32_t)idx;
            top_val[t] = l;
            if (stats) top_prob[t] = expf(l - base) / S;
        }
    }
    if (stats && t == 0) *lse = base + logf(S);
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

// Activations go through LDS up to this many columns (planes_bytes <= 52 KB).
constexpr int64_t kLdsColsMax = 16384;

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

// Largest workgroup of the kernels that run ten waves per compute unit in one
// workgroup (the gate/up wave groups, the wide lm_head shape).
constexpr int kSplitThreads = 640;

// Launch geometry in the arguments: nwg workgroups of nthr threads over
// `sweeps` sweeps, sq per workgroup and one more for the first srem.
bool set_launch(RowsArgs &a, int64_t sweeps, int64_t nwg, int nthr)
{
    if (nwg < 1 || nwg > 0x7fffffff || sweeps < 0 || sweeps > 0x7fffffff) return false;
    a.sq = (int32_t)(sweeps / nwg);
    a.srem = (int32_t)(sweeps % nwg);
    a.nwg = (int32_t)nwg;
    a.nthr = nthr;
    a.xpass = (int32_t)(((int64_t)a.nb * (kQK / 8) + nthr - 1) / nthr);
    return true;
}

template <int NMAT, int EPI, int XS, int D, int FMT = FMT_Q4K>
hipError_t launch_rows(const RowsArgs &a0, int rps, int threads, int64_t nwg, hipStream_t s,
                       int64_t nvec = 1)
{
    // Long launches (at least kIlvMinSweeps sweeps per workgroup) interleave
    // their sweeps across workgroups: lm_head 80.6 -> 78.3 us, while the
    // 2-5-sweep decode launches measured flat or slightly slower. Interleaved
    // sweeps need one buffer resource over the whole matrix (<= 1 GiB).
    RowsArgs a = a0;
    const int64_t sweeps = (a.rows + rps - 1) / rps;
    a.ilv = (Q4K_INTERLEAVE && sweeps >= kIlvMinSweeps * nwg &&
             a.rows * (int64_t)a.nb * fmt_block_bytes(FMT) <= ((int64_t)1 << 30))
                ? 1
                : 0;
    if (nvec < 1 || nvec > 65535 || !set_launch(a, sweeps, nwg, threads))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg, (unsigned)nvec), block((unsigned)threads);
    const int64_t cols = (int64_t)a.nb * kQK;
    const size_t lds = XS == XS_LDS ? (size_t)planes_bytes(cols)
                       : (a.nw && XS == XS_F32 && cols <= kNormLdsCols)
                           ? (size_t)(cols * 4 * kXPadNum / kXPadDen)
                           : 0;
    if constexpr (EPI == EPI_LOGITS && XS == XS_LDS) {
        // the wide lm_head shape: up to ten waves in one workgroup
        if (threads > 512 && threads <= kSplitThreads && rps > 1) {
            switch (rps) {
#define Q4K_RPS_CASE(R)                                                                            \
    case R:                                                                                        \
        hipLaunchKernelGGL((rows_kernel<R, NMAT, EPI, XS, kSplitThreads, D, FMT>), grid, block, lds, \
                           s, a);                                                                  \
        break;
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
    }
    if (threads > 512) {
        // only reachable with one row per sweep (cols > 32768: no LDS planes)
        if (rps != 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL((rows_kernel<1, NMAT, EPI, XS == XS_LDS ? XS_THREAD : XS, 1024, 0, FMT>),
                           grid, block, 0, s, a);
        return hipGetLastError();
    }
    switch (rps) {
#define Q4K_RPS_CASE(R)                                                                       \
    case R:                                                                                   \
        hipLaunchKernelGGL((rows_kernel<R, NMAT, EPI, XS, 512, D, FMT>), grid, block, lds, s, a); \
        break;
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

// Gate/up pair in two wave groups of one workgroup (NG = 2): 2 * threads per
// workgroup, at most kSplitThreads.

template <int EPI, int XS, int D>
hipError_t launch_rows_split(const RowsArgs &a0, int rps, int threads, int64_t nwg,
                             hipStream_t s, int64_t nvec)
{
    RowsArgs a = a0;
    const int64_t sweeps = (a.rows + rps - 1) / rps;
    a.ilv = (Q4K_INTERLEAVE && sweeps >= kIlvMinSweeps * nwg &&
             a.rows * (int64_t)a.nb * kBlockBytes <= ((int64_t)1 << 30))
                ? 1
                : 0;
    if (nvec < 1 || nvec > 65535 || 2 * threads > kSplitThreads ||
        !set_launch(a, sweeps, nwg, 2 * threads))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg, (unsigned)nvec), block((unsigned)(2 * threads));
    const int64_t cols = (int64_t)a.nb * kQK;
    const size_t lds = XS == XS_LDS ? (size_t)(2 * planes_bytes(cols)) : 0;
    switch (rps) {
#define Q4K_RPS_CASE(R)                                                                            \
    case R:                                                                                        \
        hipLaunchKernelGGL((rows_kernel<R, 2, EPI, XS, kSplitThreads, D, FMT_Q4K, 2>), grid, block, \
                           lds, s, a);                                                             \
        break;
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

// Block-floating-point activations: converted in LDS when they fit, else per
// thread.
template <int NMAT, int EPI, int D>
hipError_t launch_rows_bfp(const RowsArgs &a, int rps, int threads, int64_t nwg, hipStream_t s,
                           int64_t nvec = 1)
{
    if ((int64_t)a.nb * kQK <= kLdsColsMax)
        return launch_rows<NMAT, EPI, XS_LDS, D>(a, rps, threads, nwg, s, nvec);
    return launch_rows<NMAT, EPI, XS_THREAD, D>(a, rps, threads, nwg, s, nvec);
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

// Grid: about `per_cu` workgroups per compute unit, never more than there are
// sweeps, and enough that one workgroup's rows span less than 2^30 bytes (its
// buffer resource uses 32-bit offsets).
int64_t grid_for(int64_t rows, int64_t cols, const Shape &sh, int per_cu,
                 int block_bytes = kBlockBytes)
{
    const int64_t S = (rows + sh.rps - 1) / sh.rps;
    int64_t g = (int64_t)device_cus() * per_cu;
    const int64_t sweep_bytes = (int64_t)sh.rps * (cols / kQK) * block_bytes;
    int64_t max_sweeps = ((int64_t)1 << 30) / sweep_bytes;
    if (max_sweeps < 2) max_sweeps = 2;
    const int64_t min_g = (S + max_sweeps - 2) / (max_sweeps - 1);
    if (g < min_g) g = min_g;
    return S < g ? S : g;
}

constexpr int kLmheadWgsMax = 1024;  // bounds the candidate workspace

}  // namespace

void set_norm(RowsArgs &a, const NormIn *norm)
{
    if (!norm) return;
    a.delta = norm->delta;
    a.nw = norm->w;
    a.eps = norm->eps;
    a.h_out = norm->h_out;
}

// The f32-activation matvec launches (QKV, the short matvecs, the FFN's down
// projection): two sweeps in flight once a workgroup runs at least
// Q4K_F32_DEEP_SWEEPS of them, else one. At 2560x10240 (five per workgroup)
// two gave 6.86-6.93 us against 7.00-7.11; QKV (two per workgroup) was 0.1 us
// slower with two.
hipError_t launch_f32_store(const RowsArgs &a, const Shape &sh, int64_t nwg, hipStream_t s,
                            int64_t nvec)
{
    const int64_t sweeps = (a.rows + sh.rps - 1) / sh.rps;
    if (sweeps >= (int64_t)Q4K_F32_DEEP_SWEEPS * nwg)
        return launch_rows<1, EPI_STORE, XS_F32, 2>(a, sh.rps, sh.threads, nwg, s, nvec);
    return launch_rows<1, EPI_STORE, XS_F32, 1>(a, sh.rps, sh.threads, nwg, s, nvec);
}

hipError_t launch_rows_store(const uint8_t *W, const float *x, float *o0, float *o1, float *o2,
                             int64_t rows, int64_t cols, int64_t split0, int64_t split1,
                             hipStream_t s, const NormIn *norm, const Batch &bt)
{
    if (bt.nvec > 1 && (norm || split0 != rows)) return hipErrorInvalidValue;
    RowsArgs a = base_args(rows, cols);
    set_norm(a, norm);
    a.x_stride = bt.x_stride;
    a.o_stride = bt.o_stride;
    a.W0 = W;
    a.x = x;
    a.o0 = o0;
    a.o1 = o1;
    a.o2 = o2;
    a.split0 = split0;
    a.split1 = split1;
    const Shape sh = pick_shape(cols);
    const int64_t nwg = grid_for(rows, cols, sh, Q4K_STORE_WGS_PER_CU);
#if Q4K_STORE_F32_SWEEPS > 0
    // few sweeps per workgroup: f32 activations, no shared conversion step.
    // The conversion takes 8/RPS passes per thread (wider rows, fewer rows per
    // sweep), so the sweep count it pays off at grows with it: at 2560x10240
    // (RPS 2, 5 sweeps per workgroup) f32 7.4 us against 7.9 us, at
    // 16384x2560 (RPS 8, 8 sweeps) block floating point 8.1 us against 8.8 us.
    const int64_t sweeps = (rows + sh.rps - 1) / sh.rps;
    const int64_t f32_sweeps = (int64_t)Q4K_STORE_F32_SWEEPS * (sh.rps < 8 ? 8 / sh.rps : 1);
    if (sweeps <= f32_sweeps * nwg) return launch_f32_store(a, sh, nwg, s, bt.nvec);
#endif
    return launch_rows_bfp<1, EPI_STORE, Q4K_STORE_D>(a, sh.rps, sh.threads, nwg, s, bt.nvec);
}

hipError_t launch_gate_up(const uint8_t *Wg, const uint8_t *Wu, const float *x, float *h,
                          int64_t rows, int64_t cols, int act, hipStream_t s, const NormIn *norm,
                          const Batch &bt)
{
    if (bt.nvec > 1 && norm) return hipErrorInvalidValue;
    RowsArgs a = base_args(rows, cols);
    set_norm(a, norm);
    a.x_stride = bt.x_stride;
    a.o_stride = bt.o_stride;
    a.W0 = Wg;
    a.W1 = Wu;
    a.x = x;
    a.o0 = h;
    a.act = act;
    const Shape sh = pick_shape(cols);
    const int64_t nwg = grid_for(rows, cols, sh, Q4K_GATE_UP_WGS_PER_CU);
    if (Q4K_GATE_UP_SPLIT && 2 * sh.threads <= kSplitThreads) {
        if (cols <= kLdsColsMax)
            return launch_rows_split<EPI_GATE_UP, XS_LDS, Q4K_GATE_UP_D>(a, sh.rps, sh.threads, nwg,
                                                                         s, bt.nvec);
        return launch_rows_split<EPI_GATE_UP, XS_THREAD, Q4K_GATE_UP_D>(a, sh.rps, sh.threads, nwg,
                                                                        s, bt.nvec);
    }
    return launch_rows_bfp<2, EPI_GATE_UP, Q4K_GATE_UP_D>(a, sh.rps, sh.threads, nwg, s, bt.nvec);
}

hipError_t launch_ffn(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const float *x,
                      float *y, int64_t hidden, int64_t inter, int act, float *h, hipStream_t s,
                      const NormIn *norm, int64_t nvec)
{
    // nvec tokens: x [nvec][hidden] -> h [nvec][inter] -> y [nvec][hidden]
    hipError_t e = launch_gate_up(Wg, Wu, x, h, inter, hidden, act, s, norm,
                                  Batch{nvec, hidden, inter});
    if (e != hipSuccess) return e;
    // down projection: few rows per thread, so f32 activations (no conversion)
    RowsArgs b = base_args(hidden, inter);
    b.W0 = Wd;
    b.x = h;
    b.o0 = y;
    b.x_stride = inter;
    b.o_stride = hidden;
    const Shape sd = pick_shape(inter);
    return launch_f32_store(b, sd, grid_for(hidden, inter, sd, Q4K_DOWN_WGS_PER_CU), s, nvec);
}

hipError_t launch_q6k_matvec(const uint8_t *W, const float *x, float *y, int64_t rows,
                             int64_t cols, hipStream_t s)
{
    RowsArgs a = base_args(rows, cols);
    a.W0 = W;
    a.x = x;
    a.o0 = y;
    const Shape sh = pick_shape(cols);
    const int64_t nwg = grid_for(rows, cols, sh, Q6K_WGS_PER_CU, kQ6Bytes);
    return launch_rows<1, EPI_STORE, XS_F32, Q6K_D, FMT_Q6K>(a, sh.rps, sh.threads, nwg, s);
}

// lm_head launch shape. Wide (where it fits): twice the decode shape's rows
// per sweep in one workgroup per compute unit. Two workgroups sharing a compute
// unit do not advance together (the older one's waves are served first: on
// MI355X the second finished its rows ~8 us after the first, out of ~60 us), so
// the ten waves run as one workgroup whose waves meet at every batch barrier.
struct LmShape {
    Shape sh;
    int per_cu;
};

LmShape lmhead_shape(int64_t cols)
{
    const Shape sh = pick_shape(cols);
    if (Q4K_LMHEAD_WIDE && cols <= kLdsColsMax && 2 * sh.threads <= kSplitThreads && sh.rps <= 32)
        return {{2 * sh.rps, 2 * sh.threads}, 1};
    return {sh, Q4K_LMHEAD_WGS_PER_CU};
}

// Workgroups for at most g: enough that each holds at most kLmheadRowsPerWgMax
// rows, and no more than there are sweeps.
int64_t lmhead_grid(int64_t rows, const Shape &sh, int64_t g)
{
    // ceil(S * rps / (kLmheadRowsPerWgMax - rps)) workgroups: then none takes
    // more than kLmheadRowsPerWgMax / rps sweeps
    const int64_t S = (rows + sh.rps - 1) / sh.rps;
    const int64_t per_wg = kLmheadRowsPerWgMax - sh.rps;
    const int64_t min_g = (S * sh.rps + per_wg - 1) / per_wg;
    if (g < min_g) g = min_g;
    return S < g ? S : g;
}

int64_t lmhead_num_wgs(int64_t rows, int64_t cols)
{
    const LmShape ls = lmhead_shape(cols);
    int64_t g = (int64_t)device_cus() * ls.per_cu;
    if (g > kLmheadWgsMax) g = kLmheadWgsMax;
    return lmhead_grid(rows, ls.sh, g);
}

// The same shape with the largest grid any device uses: never below
// lmhead_num_wgs (the grid only grows with g), so it sizes the workspace.
int64_t lmhead_max_wgs(int64_t rows, int64_t cols)
{
    return lmhead_grid(rows, lmhead_shape(cols).sh, kLmheadWgsMax);
}

// lmhead_max_wgs(rows) <= kLmheadWgsMax exactly when every workgroup of that
// grid holds at most kLmheadRowsPerWgMax - rps rows of whole sweeps, i.e. when
// rows <= kLmheadWgsMax * (kLmheadRowsPerWgMax - rps) (a multiple of rps).
int64_t lmhead_rows_max(int64_t cols)
{
    const int rps = lmhead_shape(cols).sh.rps;
    return (int64_t)kLmheadWgsMax * (kLmheadRowsPerWgMax - rps);
}

hipError_t launch_lmhead_topk(const uint8_t *W, const float *x, float *logits, int64_t rows,
                              int64_t cols, int k, uint64_t *cand, int32_t *top_idx,
                              float *top_val, float2 *stats, float *top_prob, float *lse,
                              hipStream_t s)
{
    RowsArgs a = base_args(rows, cols);
    a.W0 = W;
    a.x = x;
    a.o0 = logits;
    a.cand = cand;
    a.stats = stats;
    a.k = k;
    const Shape sh = lmhead_shape(cols).sh;
    const int64_t nwg = lmhead_num_wgs(rows, cols);
    hipError_t e = launch_rows_bfp<1, EPI_LOGITS, Q4K_LMHEAD_D>(a, sh.rps, sh.threads, nwg, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(1), dim3(kMergeThreads), 0, s, cand, (int)nwg, k,
                       logits, top_idx, top_val, stats, top_prob, lse);
    return hipGetLastError();
}

}  // namespace q4k
