// Matrix-core prefill: Y[t][i] = sum_j W[i][j] X[t][j] for a batch of tokens
// on Q4_K weights, with bf16 operands and fp32 accumulation
// (v_mfma_f32_16x16x32_bf16), and the gated FFN built from it:
//   H = act(X Wg^T) * (X Wu^T)  (H rounded to bf16),  Y = H Wd^T.
//
// Sources: infer-compute README, "Quick Start" (GPU prefill for seq > 1) and
// "Shaders" table (Q4_K fused FFN row: gate+up sharing the input, gated
// GELU-tanh / SiLU, down projection); "Design Principles" item 8 (the GGUF
// Q4_K block).
//
// Operands. One MFMA multiplies a 16-token x 32-k tile of activations (A) by
// a 32-k x 16-row tile of weights (B). Lane l = n + 16c (n = l % 16,
// c = l / 16) holds eight k values of A row n and of B column n; result
// register r of lane l is D[4c + r][n] (layouts checked on MI355X).
//   * The k order inside a super-block is free as long as A and B agree. For
//     K-step j (0..7) of block b, slot i (0..7) of lane group c is element
//         e(j, c, i) = 64c + 32*(j/4) + 8*(j%4) + i
//     of the block. Lane group c then only needs quant bytes 32c..32c+31 of the
//     row (all of sub-blocks 2c and 2c+1): K-steps 0..3 are their low nibbles,
//     4..7 their high nibbles.
//   * Activations are converted once to bf16 (round to nearest even) in that
//     order, "fragment-major": 16-byte pieces indexed
//         (((tg * KB + b) * 8 + j) * 4 + tt) * 64 + (m + 16c)
//     for token 64 tg + 16 tt + m. One super-block column of a 64-token group
//     is then 32 KB of consecutive bytes, and each 1 KB is one MFMA operand.
//   * Weights are dequantised in f32 (w = d sc q - dmin m, one fused
//     multiply-add: the product and the sum are exact before the single
//     rounding, so w equals the correctly rounded f32 weight), then rounded to
//     bf16 straight into the B operand registers.
//
// Work decomposition. A workgroup owns n_t = 4A + B tiles of 16 weight rows
// (for the gate/up pair a tile is 8 gate rows and the same 8 up rows) over a
// range of super-blocks (a K split), for 64 tokens. Eight compute waves, two
// per SIMD, run in lockstep over the super-blocks; the two waves of SIMD s
// (waves s and s + 4) split every super-block's K-steps by quant-byte half, so
// they dequantise disjoint weights and add their partial sums at the end:
//   * tiles 0..4A-1 are "own" tiles: the pair of SIMD s dequantises tiles
//     sA..sA+A-1 into its registers and multiplies them by all four token
//     tiles;
//   * tiles 4A..4A+B-1 are "shared": all 512 compute threads dequantise them
//     into LDS (bf16), and the pair of SIMD s multiplies them by token tile s.
// Every SIMD then dequantises the same number of weights and issues the same
// number of MFMAs, whatever n_t is, so one workgroup per CU keeps all four
// SIMDs equally busy. A ninth wave only copies the activation fragments (and,
// where they fit, the weight bytes) of the next super-blocks into LDS rings
// with LDS-DMA loads; its wait counter is its own, so the compute waves never
// wait on its loads except through the per-super-block barrier.
//
// K splits write f32 partial sums; a second kernel adds them in a fixed order
// (and applies the gated activation for the gate/up pair). Results are
// deterministic: no atomics, one writer per element.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_internal.h"

namespace q4k {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // plain vector: no struct copies
typedef __attribute__((address_space(3))) void *lds_ptr;

constexpr int kTokGroup = 64;          // tokens per group (four 16-token tiles)
constexpr int kChunk = 32768;          // bytes of one super-block column of a token group
constexpr int kXBufs = 3;              // activation chunks in the LDS ring
constexpr int kRing = 3;               // weight register ring slots (2 super-blocks in flight; deeper
                                       // rings measured slower: the extra loads congest the CU)
constexpr int kComputeWaves = 8;       // two per SIMD
constexpr int kComputeThreads = 64 * kComputeWaves;
constexpr int kThreads = kComputeThreads + 64;   // + one loader wave
constexpr int kTileBytesPerBlock = 16 * kBlockBytes;

// A launch plan: tiles of 16 weight rows per workgroup (n_t), the K split (S
// splits of kps super-blocks), the row groups (rg) and the 64-token groups (tg).
struct MmPlan {
    int n_t, S, kps;
    int64_t rg, tg;
};

struct MmArgs {
    const uint8_t *W0;     // weights (gate matrix of the pair)
    const uint8_t *W1;     // up matrix of the pair (unused for one matrix)
    const uint8_t *Xf;     // bf16 activation fragments, KB = nb super-blocks per token group
    void *out;             // one matrix: Y f32 [seq][rows]; the pair: H as bf16 fragments (KB = out_kb)
    float *partial;        // K splits: f32 [S][seq][NMAT*rows]
    int32_t rows;          // rows per matrix
    int32_t nb;            // super-blocks per weight row
    int32_t seq;
    int32_t n_tiles;       // tiles per workgroup (4A + B)
    int32_t S;             // K splits
    int32_t kps;           // super-blocks per split
    int32_t act;
    int32_t out_kb;
};

// Gated activations as z * sigmoid(k): GELU-tanh has k = 2 sqrt(2/pi) (z +
// 0.044715 z^3), since 0.5 z (1 + tanh(y)) = z / (1 + e^(-2y)); SiLU has k = z.
// One exponential and one reciprocal; the result is rounded to bf16 next.
__device__ __forceinline__ float act_apply(float z, int act)
{
    const float k = act == 0 ? 1.5957691216057308f * (z + 0.044715f * z * z * z) : z;
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-k));
}

// Byte offset of (token, k) in a fragment-major bf16 activation buffer with
// KB super-blocks per token group.
__device__ __forceinline__ int64_t frag_offset(int64_t token, int64_t k, int64_t KB)
{
    const int64_t tg = token >> 6;
    const int tt = (int)(token >> 4) & 3, m = (int)token & 15;
    const int64_t kb = k >> 8;
    const int e = (int)k & 255, c = e >> 6, r = e & 63;
    const int j = ((r >> 5) << 2) | ((r & 31) >> 3), i = r & 7;
    return (((((tg * KB + kb) * 8 + j) * 4 + tt) * 64) + m + 16 * c) * 16 + 2 * i;
}

// An AND the compiler cannot see through: without it the mask and the
// following byte conversions are fused into bit-field extracts, one more
// instruction per weight.
__device__ __forceinline__ uint32_t and_opaque(uint32_t v, uint32_t m)
{
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(m), "v"(v));
    return r;
}

// Dequantisation coefficients of sub-blocks 2g (low nibbles) and 2g+1 (high
// nibbles) of a block with header h: w = a*q + b. The high-nibble factor is
// pre-divided by 16 because those nibbles are used in place (bits 4..7).
struct Coef {
    float a_lo, b_lo, a_hi, b_hi;
};

__device__ __forceinline__ Coef block_coef(uint4 h, int g)
{
    const float d = __half2float(__ushort_as_half((unsigned short)(h.x & 0xFFFFu)));
    const float dmin = __half2float(__ushort_as_half((unsigned short)(h.x >> 16)));
    // The 12 scale bytes s[0..11] are h.y (s[0..3]), h.z (s[4..7]), h.w
    // (s[8..11]). Sub-blocks 2g and 2g+1 use the byte pair 2(g%2), 2(g%2)+1 of
    // each word; for g < 2 the 6-bit values are the low bits of s[2g+e] and
    // s[2g+4+e], for g >= 2 they are nibbles of s[2g+4+e] with the top two
    // bits of s[2g-4+e] (scale) and s[2g+e] (min).
    const uint32_t sh = (uint32_t)(g & 1) << 4;
    const uint32_t P = h.y >> sh, Q = h.z >> sh, R = h.w >> sh;
    const uint32_t sc_lo6 = P & 0x3F3Fu, m_lo6 = Q & 0x3F3Fu;
    const uint32_t sc_hi6 = (R & 0x0F0Fu) | ((P >> 2) & 0x3030u);
    const uint32_t m_hi6 = ((R >> 4) & 0x0F0Fu) | ((Q >> 2) & 0x3030u);
    const uint32_t SC = g < 2 ? sc_lo6 : sc_hi6;
    const uint32_t M = g < 2 ? m_lo6 : m_hi6;
    Coef k;
    k.a_lo = d * (float)(SC & 0xFFu);
    k.b_lo = -dmin * (float)(M & 0xFFu);
    k.a_hi = d * 0.0625f * (float)((SC >> 8) & 0xFFu);
    k.b_hi = -dmin * (float)((M >> 8) & 0xFFu);
    return k;
}

// Two f32 values -> one word of two bf16 (round to nearest even; the first
// value in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

// Eight weights from two quant words: the low (HI = false) or high nibbles
// of bytes 0..3 of w0 then of w1, rounded to bf16.
template <bool HI>
__device__ __forceinline__ bf16x8 deq8(uint32_t w0, uint32_t w1, float a, float b)
{
    const uint32_t mask = HI ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
    const uint32_t u0 = and_opaque(w0, mask), u1 = and_opaque(w1, mask);
    uint4 r;
    r.x = pack_bf16(fmaf(a, (float)(u0 & 0xFFu), b), fmaf(a, (float)((u0 >> 8) & 0xFFu), b));
    r.y = pack_bf16(fmaf(a, (float)((u0 >> 16) & 0xFFu), b), fmaf(a, (float)(u0 >> 24), b));
    r.z = pack_bf16(fmaf(a, (float)(u1 & 0xFFu), b), fmaf(a, (float)((u1 >> 8) & 0xFFu), b));
    r.w = pack_bf16(fmaf(a, (float)((u1 >> 16) & 0xFFu), b), fmaf(a, (float)(u1 >> 24), b));
    return __builtin_bit_cast(bf16x8, r);
}

// LDS position (16-byte units) of the B operand of lane n + 16c at K-step j
// inside one 1 KB operand: a permutation within lane group c chosen so that
// the 16 threads that dequantise one row's 16 quant pieces write 16 different
// bank groups.
__device__ __forceinline__ int b_pos(int n, int c, int j)
{
    return 16 * c + (n ^ ((j & 3) | (c << 2)));
}

// Weight bytes of one super-block for a workgroup of NT tiles (16 rows each),
// and whether the LDS weight ring (three of them) fits beside the activation
// ring and the shared-tile operand buffers.
constexpr int w_stage_bytes(int nt) { return nt * 16 * kBlockBytes; }
constexpr int b_buf_bytes(int b) { return b > 0 ? 2 * b * 8192 : 16; }
constexpr bool lds_weights(int a, int b)
{
    // LDS budget, and the loader's prologue (two weight stages and one
    // activation chunk of 32 loads) within the 63 outstanding loads of a wave
    return kXBufs * kChunk + b_buf_bytes(b) + 3 * w_stage_bytes(4 * a + b) <= 160 * 1024 - 2048 &&
           2 * ((w_stage_bytes(4 * a + b) / 16 + 63) / 64) + kChunk / 1024 <= 63;
}

// s_waitcnt vmcnt(N) for a compile-time N <= 63 (expcnt / lgkmcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_vmcnt_le(int n)
{
    // s_waitcnt with expcnt / lgkmcnt at their maxima (no wait on them).
    if (n >= 32)
        __builtin_amdgcn_s_waitcnt(0x8F70);   // vmcnt(32)
    else
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
}

// Workgroup barrier that neither waits for outstanding global loads nor lets
// the compiler move memory accesses across it.
__device__ __forceinline__ void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Weight loads of one super-block, per thread: own tiles (header + the 16
// quant bytes of this wave's half of the lane's 32-byte group) and shared
// tiles (header + 4 quant bytes).
template <int A, int B>
struct Slot {
    uint4 oh[A > 0 ? A : 1], oq[A > 0 ? A : 1];
    uint4 sh[B > 0 ? B : 1];
    uint32_t sq[B > 0 ? B : 1];
};

// LDS operands of one K-step: the four token tiles, rotated so that xa[0] is
// this SIMD's own token tile (the shared tiles' operand), and the shared
// tiles' weights.
template <int B>
struct Ops {
    bf16x8 xa[4];
    bf16x8 wb[B > 0 ? B : 1];
};

template <int NMAT>
__device__ __forceinline__ const uint8_t *row_ptr(const MmArgs &p, int64_t tile, int nn)
{
    int64_t row;
    const uint8_t *base;
    if (NMAT == 1) {
        row = 16 * tile + nn;
        base = p.W0;
    } else {
        row = 8 * tile + (nn & 7);
        base = nn < 8 ? p.W0 : p.W1;
    }
    // Rows past the end read the last row; their results are never stored.
    row = row < p.rows ? row : (int64_t)p.rows - 1;
    return base + row * (int64_t)p.nb * kBlockBytes;
}

// Four weights from one quant word: low (HI = false) or high nibbles of bytes
// 0..3, rounded to bf16, as two words.
template <bool HI>
__device__ __forceinline__ uint2 deq4(uint32_t w, float a, float b)
{
    const uint32_t u = and_opaque(w, HI ? 0xF0F0F0F0u : 0x0F0F0F0Fu);
    uint2 r;
    r.x = pack_bf16(fmaf(a, (float)(u & 0xFFu), b), fmaf(a, (float)((u >> 8) & 0xFFu), b));
    r.y = pack_bf16(fmaf(a, (float)((u >> 16) & 0xFFu), b), fmaf(a, (float)(u >> 24), b));
    return r;
}

// The matrix-core kernel. Waves 0..7 compute: SIMD s = wave % 4 runs waves s
// and s + 4, which split every super-block's eight K-steps by quant-byte half
// (half h covers bytes 16h..16h+15 of each 32-byte group: K-steps 2h, 2h+1 of
// the low nibbles and 4+2h, 5+2h of the high nibbles), so the two waves of a
// SIMD dequantise disjoint weights; their partial sums are added at the end.
// Wave 8 is the loader: it copies the activation chunks of the next
// super-blocks into a 3-deep LDS ring with LDS-DMA loads, on a wait counter
// of its own. Where it fits (LDS, and the loader's 63 outstanding loads) it
// also copies each super-block's weight bytes into a 3-deep LDS ring and the
// compute waves issue no global loads; otherwise they prefetch their weights
// into a register ring of kRing - 1 super-blocks. One barrier per super-block.
template <int NMAT, int A, int B>
__global__ __launch_bounds__(kThreads, 1) void mm_kernel(MmArgs p)
{
    // With kWL the loader also copies each super-block's weight bytes (all of
    // the workgroup's rows, 144 B each, in tile-row order) into a 3-deep LDS
    // ring, so the compute waves issue no global loads at all.
    constexpr int NT = 4 * A + B;
    constexpr bool kWL = lds_weights(A, B);
    constexpr int kWStage = w_stage_bytes(NT);
    constexpr int kWPieces = NT * 16 * (kBlockBytes / 16);   // 16-byte pieces per stage
    constexpr int kWInstr = (kWPieces + 63) / 64;            // loader instructions per stage
    __shared__ __attribute__((aligned(16))) uint8_t xbuf[kXBufs * kChunk];
    __shared__ __attribute__((aligned(16))) uint8_t bbuf[b_buf_bytes(B)];
    __shared__ __attribute__((aligned(16))) uint8_t wbuf[kWL ? 3 * kWStage : 16];

    const int rg = blockIdx.x / p.S, sp = blockIdx.x % p.S;
    const int64_t tg = blockIdx.y;
    const int kb0 = sp * p.kps;
    const int nblk = min(p.nb, kb0 + p.kps) - kb0;
    const int niter = (nblk + kRing - 1) / kRing * kRing;
    const int64_t tile0 = (int64_t)rg * p.n_tiles;
    const int t = threadIdx.x;
    const int wave = t >> 6, l = t & 63;

    if (wave == kComputeWaves) {
        // Loader: chunk b (activations of super-block kb0 + b) -> xbuf[b % 3].
        const uint8_t *src = p.Xf + ((int64_t)tg * p.nb + kb0) * kChunk + l * 16;
        auto issue = [&](int b) {
            const uint8_t *s = src + (int64_t)b * kChunk;
            uint8_t *dst = xbuf + (b % kXBufs) * kChunk;
#pragma unroll
            for (int i = 0; i < kChunk / 1024; ++i)
                __builtin_amdgcn_global_load_lds((const void *)(s + i * 1024),
                                                 (lds_ptr)(dst + i * 1024), 16, 0, 0);
        };
        if constexpr (kWL) {
            // Weights of block b go out before its activations, so that at
            // barrier b only the activations of block b+1 may be in flight:
            // block b+1's weights (staged for the shared tiles at the end of
            // block b) have landed with block b's activations.
            auto issue_w = [&](int b) {
                const int64_t boff = (int64_t)(kb0 + b) * kBlockBytes;
                uint8_t *dst = wbuf + (b % 3) * kWStage;
#pragma unroll
                for (int i = 0; i < kWInstr; ++i) {
                    const int pc = i * 64 + l;
                    if (pc < kWPieces) {
                        const int row = pc / 9, piece = pc % 9;
                        const uint8_t *srcw = row_ptr<NMAT>(p, tile0 + row / 16, row % 16) + boff + piece * 16;
                        __builtin_amdgcn_global_load_lds((const void *)srcw, (lds_ptr)(dst + i * 1024), 16, 0, 0);
                    }
                }
            };
            // prologue: weights of blocks 0 and 1, then activations of block
            // 0; once both weight stages have landed (only block 0's
            // activations may still be in flight) the shared tiles of block 0
            // can be staged, and block 1's activations go out. At most
            // 2 * kWInstr + 32 <= 63 loads are outstanding here.
            static_assert(2 * kWInstr + kChunk / 1024 <= 63, "loader wait counter");
            issue_w(0);
            if (nblk > 1) issue_w(1);
            issue(0);
            wait_vmcnt<kChunk / 1024>();
            barrier_lds();
            if (nblk > 1) issue(1);
            for (int b = 0; b < niter; ++b) {
                if (b < nblk) wait_vmcnt_le(b + 1 < nblk ? 32 : 0);
                barrier_lds();
                if (b + 2 < nblk) {
                    issue_w(b + 2);
                    issue(b + 2);
                }
            }
        } else {
            issue(0);
            if (nblk > 1) issue(1);
            for (int b = 0; b < niter; ++b) {
                if (b < nblk) wait_vmcnt_le(b + 1 < nblk ? 32 : 0);   // chunk b has landed
                barrier_lds();
                if (b + 2 < nblk) issue(b + 2);   // into the buffer chunk b-1 used
            }
        }
        barrier_lds();   // the compute waves' two barriers of the pair reduction
        barrier_lds();
        return;
    }

    const int n = l & 15, c = l >> 4;
    const int simd = wave & 3, half = wave >> 2;
    const int ns = t >> 5, q4 = t & 31;      // shared-tile dequant: row ns, quant word q4
    const uint8_t *rp_own[A > 0 ? A : 1];
    const uint8_t *rp_sh[B > 0 ? B : 1];
#pragma unroll
    for (int i = 0; i < A; ++i) rp_own[i] = row_ptr<NMAT>(p, tile0 + simd * A + i, n);
#pragma unroll
    for (int s = 0; s < B; ++s) rp_sh[s] = row_ptr<NMAT>(p, tile0 + 4 * A + s, ns);

    Slot<A, B> ring[kRing];
    // kWL: block b's weight bytes in the LDS ring; row rr of the workgroup
    // (tile rr / 16, tile row rr % 16) starts at byte 144 rr of the stage.
    auto wrow = [&](int b, int rr) -> const uint8_t * {
        return wbuf + (b % 3) * kWStage + rr * kBlockBytes;
    };
    auto load_own_lds = [&](Slot<A, B> &sl, int b) {
#pragma unroll
        for (int i = 0; i < A; ++i) {
            const uint8_t *r = wrow(b, (simd * A + i) * 16 + n);
            sl.oh[i] = *reinterpret_cast<const uint4 *>(r);
            sl.oq[i] = *reinterpret_cast<const uint4 *>(r + 16 + 32 * c + 16 * half);
        }
    };
    auto load_sh_lds = [&](Slot<A, B> &sl, int b) {
#pragma unroll
        for (int s = 0; s < B; ++s) {
            const uint8_t *r = wrow(b, (4 * A + s) * 16 + ns);
            sl.sh[s] = *reinterpret_cast<const uint4 *>(r);
            sl.sq[s] = *reinterpret_cast<const uint32_t *>(r + 16 + 4 * q4);
        }
    };
    auto load = [&](Slot<A, B> &sl, int b) {
        const int64_t off = (int64_t)(kb0 + min(b, nblk - 1)) * kBlockBytes;
#pragma unroll
        for (int i = 0; i < A; ++i) {
            const uint8_t *r = rp_own[i] + off;
            sl.oh[i] = *reinterpret_cast<const uint4 *>(r);
            sl.oq[i] = *reinterpret_cast<const uint4 *>(r + 16 + 32 * c + 16 * half);
        }
#pragma unroll
        for (int s = 0; s < B; ++s) {
            const uint8_t *r = rp_sh[s] + off;
            sl.sh[s] = *reinterpret_cast<const uint4 *>(r);
            sl.sq[s] = *reinterpret_cast<const uint32_t *>(r + 16 + 4 * q4);
        }
    };
    // Shared tiles of one block -> LDS operand buffer `buf`. Thread (ns, q4)
    // owns quant bytes 4q4..4q4+3 of a shared row: group g = q4/8, K-step
    // (q4%8)/2 (low nibbles; +4 for the high ones), elements 4(q4%2)..+3 of
    // that slot.
    auto stage = [&](const Slot<A, B> &sl, int buf) {
#pragma unroll
        for (int s = 0; s < B; ++s) {
            const int g = q4 >> 3, jl = (q4 & 7) >> 1, sub = q4 & 1;
            const Coef k = block_coef(sl.sh[s], g);
            uint8_t *base = bbuf + (buf * B + s) * 8192 + 8 * sub;
            *reinterpret_cast<uint2 *>(base + (jl * 64 + b_pos(ns, g, jl)) * 16) =
                deq4<false>(sl.sq[s], k.a_lo, k.b_lo);
            *reinterpret_cast<uint2 *>(base + ((jl + 4) * 64 + b_pos(ns, g, jl + 4)) * 16) =
                deq4<true>(sl.sq[s], k.a_hi, k.b_hi);
        }
    };

    f32x4 acc[A > 0 ? A : 1][4];     // own tile i, token tile (simd + tt) % 4
    f32x4 acc_sh[B > 0 ? B : 1];     // shared tile s, token tile simd
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[i][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < B; ++s) acc_sh[s] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (kWL) {
        barrier_lds();   // the loader has block 0's (and 1's) weights in LDS
        if constexpr (B > 0) {
            load_sh_lds(ring[0], 0);
            stage(ring[0], 0);
        }
    } else {
#pragma unroll
        for (int b = 0; b < kRing - 1; ++b) load(ring[b], b);
        // Keep all prologue loads ahead of the first wait (the scheduler would
        // otherwise issue blocks 1.. only after block 0 has arrived).
        asm volatile("" ::: "memory");
        if constexpr (B > 0) stage(ring[0], 0);
    }

    for (int b0 = 0; b0 < niter; b0 += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int b = b0 + u;
            barrier_lds();   // block b's activations and shared operands are in LDS
            if constexpr (kWL) {
                if (b < nblk) load_own_lds(ring[u], b);
            } else {
                load(ring[(u + kRing - 1) % kRing], b + kRing - 1);
            }
            if (b < nblk) {
                const uint8_t *xb = xbuf + (b % kXBufs) * kChunk;
                const uint8_t *sbase = bbuf + ((b & 1) * B) * 8192;
                const Slot<A, B> &sl = ring[u];
                Coef k[A > 0 ? A : 1];
#pragma unroll
                for (int i = 0; i < A; ++i) k[i] = block_coef(sl.oh[i], c);
                // this wave's K-steps: jj = 0, 1 low nibbles, 2, 3 high nibbles
                auto kstep = [&](int jj) { return (jj < 2 ? 0 : 4) + 2 * half + (jj & 1); };
                // LDS operands of the next K-step are requested before the
                // current one is dequantised and multiplied.
                auto read_ops = [&](int jj, Ops<B> &o) {
                    const int j = kstep(jj);
                    if constexpr (A > 0) {
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt)
                            o.xa[tt] = *reinterpret_cast<const bf16x8 *>(
                                xb + ((j * 4 + ((simd + tt) & 3)) * 64 + l) * 16);
                    } else {
                        o.xa[0] = *reinterpret_cast<const bf16x8 *>(xb + ((j * 4 + simd) * 64 + l) * 16);
                    }
                    if constexpr (B > 0) {
#pragma unroll
                        for (int s = 0; s < B; ++s)
                            o.wb[s] = *reinterpret_cast<const bf16x8 *>(sbase + s * 8192 + (j * 64 + b_pos(n, c, j)) * 16);
                    }
                };
                Ops<B> ops[2];
                read_ops(0, ops[0]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    if (jj + 1 < 4) read_ops(jj + 1, ops[(jj + 1) & 1]);
                    const Ops<B> &o = ops[jj & 1];
#pragma unroll
                    for (int i = 0; i < A; ++i) {
                        const uint4 &qa = sl.oq[i];
                        const uint32_t w0 = (jj & 1) ? qa.z : qa.x, w1 = (jj & 1) ? qa.w : qa.y;
                        const bf16x8 wb = jj < 2 ? deq8<false>(w0, w1, k[i].a_lo, k[i].b_lo)
                                                 : deq8<true>(w0, w1, k[i].a_hi, k[i].b_hi);
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt)
                            acc[i][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.xa[tt], wb, acc[i][tt], 0, 0, 0);
                    }
#pragma unroll
                    for (int s = 0; s < B; ++s)
                        acc_sh[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.xa[0], o.wb[s], acc_sh[s], 0, 0, 0);
                }
                if constexpr (B > 0) {
                    if (b + 1 < nblk) {
                        if constexpr (kWL) load_sh_lds(ring[(u + 1) % kRing], b + 1);
                        stage(ring[(u + 1) % kRing], (b + 1) & 1);
                    }
                }
            }
        }
    }

    // ---- the two halves of each SIMD add up (through LDS, reusing xbuf) ----
    constexpr int NACC = 16 * A + 4 * B;
    float *red = reinterpret_cast<float *>(xbuf) + simd * NACC * 64 + l;
    barrier_lds();                                  // everyone is done with xbuf
    if (half == 1) {
#pragma unroll
        for (int i = 0; i < A; ++i)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[((i * 4 + tt) * 4 + r) * 64] = acc[i][tt][r];
#pragma unroll
        for (int s = 0; s < B; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(16 * A + 4 * s + r) * 64] = acc_sh[s][r];
    }
    barrier_lds();
    if (half == 1) return;
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][tt][r] += red[((i * 4 + tt) * 4 + r) * 64];
#pragma unroll
    for (int s = 0; s < B; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc_sh[s][r] += red[(16 * A + 4 * s + r) * 64];

    // ---- epilogue: lane (n, c), register r -> token tok0 + 4c + r, tile row n ----
    const bool split = p.S > 1;
    const int64_t tok_base = tg * kTokGroup;
    auto store = [&](f32x4 v, int64_t tile, int ttile) {
        const int64_t tok0 = tok_base + 16 * ttile;
        if (NMAT == 2 && !split) {
            // gated activation: lanes n < 8 hold the gate rows, n >= 8 the up
            // rows; a row rotation by 8 pairs them. Lanes n < 8 finish
            // registers 0, 1, lanes n >= 8 registers 2, 3.
            float other[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                other[r] = __int_as_float(
                    __builtin_amdgcn_update_dpp(0, __float_as_int(v[r]), 0x128, 0xF, 0xF, false));
            const int64_t irow = 8 * tile + (n & 7);
            if (irow < p.rows) {
                const int64_t kb = irow >> 8;
                const int e = (int)irow & 255, cc = e >> 6, rr = e & 63;
                const int j = ((rr >> 5) << 2) | ((rr & 31) >> 3), ii = rr & 7;
                // fragment offset of (tok0 + 4c, irow); + 16 bytes per token
                uint8_t *hb = (uint8_t *)p.out +
                              ((((tg * p.out_kb + kb) * 8 + j) * 4 + ttile) * 64 + 4 * c + 16 * cc) * 16 + 2 * ii;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int r = (n < 8 ? 0 : 2) + h2;
                    const float g = n < 8 ? v[r] : other[r];
                    const float u = n < 8 ? other[r] : v[r];
                    *reinterpret_cast<__bf16 *>(hb + r * 16) = (__bf16)(act_apply(g, p.act) * u);
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t token = tok0 + 4 * c + r;
                if (token >= p.seq) continue;
                int64_t col, ncols;
                if (NMAT == 1) {
                    col = 16 * tile + n;
                    ncols = p.rows;
                    if (col >= p.rows) continue;
                } else {
                    const int64_t irow = 8 * tile + (n & 7);
                    if (irow >= p.rows) continue;
                    col = n < 8 ? irow : (int64_t)p.rows + irow;
                    ncols = 2 * (int64_t)p.rows;
                }
                float *o = split ? p.partial + (int64_t)sp * p.seq * ncols : (float *)p.out;
                o[token * ncols + col] = v[r];
            }
        }
    };
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) store(acc[i][tt], tile0 + simd * A + i, (simd + tt) & 3);
#pragma unroll
    for (int s = 0; s < B; ++s) store(acc_sh[s], tile0 + 4 * A + s, simd);
}

// f32 activations [seq][cols] -> bf16 fragments; zeros for the padding
// tokens of the last group. Thread = 8 consecutive values of one token (reads
// are row-contiguous), written to their 16-byte fragment piece.
__global__ __launch_bounds__(256) void x_to_frag_kernel(const float *X, uint8_t *Xf, int64_t seq,
                                                         int64_t seq_pad, int64_t cols)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t k8n = cols >> 3;
    if (idx >= seq_pad * k8n) return;
    const int64_t token = idx / k8n, k0 = (idx % k8n) * 8;
    bf16x8 v;
    if (token < seq) {
        const float4 a = *reinterpret_cast<const float4 *>(X + token * cols + k0);
        const float4 b = *reinterpret_cast<const float4 *>(X + token * cols + k0 + 4);
        v[0] = (__bf16)a.x; v[1] = (__bf16)a.y; v[2] = (__bf16)a.z; v[3] = (__bf16)a.w;
        v[4] = (__bf16)b.x; v[5] = (__bf16)b.y; v[6] = (__bf16)b.z; v[7] = (__bf16)b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.0f;
    }
    *reinterpret_cast<bf16x8 *>(Xf + frag_offset(token, k0, cols >> 8)) = v;
}

constexpr int kReduceBatch = 8;   // split loads in flight per thread

// K splits: Y[t][i] = sum_s P[s][t][i], s in order; a batch of splits' loads
// is issued before its sums.
__global__ __launch_bounds__(256) void reduce_y_kernel(const float *P, float *Y, int64_t n, int S)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = P[i];
    for (int s0 = 1; s0 < S; s0 += kReduceBatch) {
        float v[kReduceBatch];
#pragma unroll
        for (int k = 0; k < kReduceBatch; ++k)
            if (s0 + k < S) v[k] = P[(int64_t)(s0 + k) * n + i];
#pragma unroll
        for (int k = 0; k < kReduceBatch; ++k)
            if (s0 + k < S) acc += v[k];
    }
    Y[i] = acc;
}

// The same, four consecutive outputs per thread (n % 4 == 0, Y 16-byte
// aligned): one 16-byte load per split, all issued before the sums.
__global__ __launch_bounds__(256) void reduce_y4_kernel(const float4 *P, float4 *Y, int64_t n4, int S)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    float4 acc = P[i];
    for (int s0 = 1; s0 < S; s0 += kReduceBatch) {
        float4 v[kReduceBatch];
#pragma unroll
        for (int k = 0; k < kReduceBatch; ++k)
            if (s0 + k < S) v[k] = P[(int64_t)(s0 + k) * n4 + i];
#pragma unroll
        for (int k = 0; k < kReduceBatch; ++k)
            if (s0 + k < S) {
                acc.x += v[k].x;
                acc.y += v[k].y;
                acc.z += v[k].z;
                acc.w += v[k].w;
            }
    }
    Y[i] = acc;
}

// K splits of the gate/up pair: P[s][t][0..2 inter) -> H = act(G) * U as bf16
// fragments for every token of the padded groups (zeros past seq).
__global__ __launch_bounds__(256) void reduce_gated_kernel(const float *P, uint8_t *Hf, int64_t seq,
                                                           int64_t seq_pad, int64_t inter, int S,
                                                           int act)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= seq_pad * inter) return;
    const int64_t token = idx / inter, i = idx % inter;
    float h = 0.0f;
    if (token < seq) {
        const int64_t stride = seq * 2 * inter;
        const float *pg = P + token * 2 * inter + i;
        float g = pg[0], u = pg[inter];
        for (int s0 = 1; s0 < S; s0 += kReduceBatch) {   // a batch of loads, then its sums
            float vg[kReduceBatch], vu[kReduceBatch];
#pragma unroll
            for (int k = 0; k < kReduceBatch; ++k)
                if (s0 + k < S) {
                    vg[k] = pg[(s0 + k) * stride];
                    vu[k] = pg[(s0 + k) * stride + inter];
                }
#pragma unroll
            for (int k = 0; k < kReduceBatch; ++k)
                if (s0 + k < S) {
                    g += vg[k];
                    u += vu[k];
                }
        }
        h = act_apply(g, act) * u;
    }
    *reinterpret_cast<__bf16 *>(Hf + frag_offset(token, i, inter >> 8)) = (__bf16)h;
}

// ------------------------------------------------------------------ host ---

int device_cus_mm()
{
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cache[dev] = v;
    }
    return cache[dev];
}

constexpr int kMaxTilesPerWg = 6;   // 7 and 8 tiles spill registers

// Tiles per workgroup and K split for T tiles of nb super-blocks and TG token
// groups: minimise the per-CU weight stream of the slowest round plus a charge
// for the partial sums a split writes and reads back.
MmPlan plan_for(int64_t T, int nb, int64_t seq, int64_t rows_out, int cus)
{
    const int64_t TG = (seq + kTokGroup - 1) / kTokGroup;
    MmPlan best{};
    double best_cost = -1.0;
    for (int s_try = 1; s_try <= nb; ++s_try) {
        const int kps = (nb + s_try - 1) / s_try;
        const int S = (nb + kps - 1) / kps;
        if (S != s_try) continue;
        int64_t rg_target = cus / ((int64_t)S * TG);
        if (rg_target < 1) rg_target = 1;
        int64_t n_t = (T + rg_target - 1) / rg_target;
        if (n_t > kMaxTilesPerWg) n_t = kMaxTilesPerWg;
        if (n_t < 1) n_t = 1;
        const int64_t rg = (T + n_t - 1) / n_t;
        const int64_t wgs = rg * S * TG;
        const int64_t rounds = (wgs + cus - 1) / cus;
        // per-CU bytes of the slowest round: weights from HBM, plus the
        // activation chunks (32 KB per super-block and token group, from L2,
        // charged at half weight)
        double cost = (double)rounds * (double)kps * ((double)n_t * kTileBytesPerBlock + 0.5 * kChunk) * cus;
        // a split writes and re-reads partial sums and costs a second kernel
        // (about 3 us of launch and latency, charged as bytes at 6 TB/s)
        if (S > 1) cost += 0.35 * (double)S * (double)seq * (double)rows_out * 8.0 + 18e6;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best.n_t = (int)n_t;
            best.S = S;
            best.kps = kps;
            best.rg = rg;
            best.tg = TG;
        }
    }
    return best;
}

template <int NMAT, int A, int B>
hipError_t launch_mm_t(const MmArgs &a, const MmPlan &pl, hipStream_t s)
{
    hipLaunchKernelGGL((mm_kernel<NMAT, A, B>), dim3((unsigned)(pl.rg * pl.S), (unsigned)pl.tg),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int NMAT>
hipError_t launch_mm(const MmArgs &a, const MmPlan &pl, hipStream_t s)
{
    switch (pl.n_t) {
        case 1: return launch_mm_t<NMAT, 0, 1>(a, pl, s);
        case 2: return launch_mm_t<NMAT, 0, 2>(a, pl, s);
        case 3: return launch_mm_t<NMAT, 0, 3>(a, pl, s);
        case 4: return launch_mm_t<NMAT, 1, 0>(a, pl, s);
        case 5: return launch_mm_t<NMAT, 1, 1>(a, pl, s);
        case 6: return launch_mm_t<NMAT, 1, 2>(a, pl, s);
        case 7: return launch_mm_t<NMAT, 1, 3>(a, pl, s);
        case 8: return launch_mm_t<NMAT, 2, 0>(a, pl, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_x_to_frag(const float *X, uint8_t *Xf, int64_t seq, int64_t cols, hipStream_t s)
{
    const int64_t seq_pad = (seq + kTokGroup - 1) / kTokGroup * kTokGroup;
    const int64_t n = seq_pad * (cols / 8);
    hipLaunchKernelGGL(x_to_frag_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, X, Xf,
                       seq, seq_pad, cols);
    return hipGetLastError();
}

int64_t up256(int64_t v) { return (v + 255) / 256 * 256; }
int64_t partial_bytes(const MmPlan &pl, int64_t seq, int64_t rows, int nmat)
{
    return pl.S > 1 ? (int64_t)pl.S * seq * rows * nmat * 4 : 0;
}

MmPlan plan_of(int64_t rows, int64_t cols, int64_t seq, int nmat)
{
    const int64_t T = nmat == 1 ? (rows + 15) / 16 : (rows + 7) / 8;
    return plan_for(T, (int)(cols / 256), seq, rows * nmat, device_cus_mm());
}

int64_t frag_bytes(int64_t seq, int64_t cols)
{
    return (seq + kTokGroup - 1) / kTokGroup * kTokGroup * cols * 2;
}

hipError_t launch_reduce_y(const float *P, float *Y, int64_t n, int S, hipStream_t s)
{
    if (n % 4 == 0 && ((uintptr_t)Y & 15) == 0) {
        const int64_t n4 = n / 4;
        hipLaunchKernelGGL(reduce_y4_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                           (const float4 *)P, (float4 *)Y, n4, S);
    } else {
        hipLaunchKernelGGL(reduce_y_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, P,
                           Y, n, S);
    }
    return hipGetLastError();
}

}  // namespace

// Workspace of the matrix product: activation fragments | partial sums of a
// K split (each piece 256-byte aligned).
int64_t mm_matmul_workspace(int64_t rows, int64_t cols, int64_t seq)
{
    const MmPlan pl = plan_of(rows, cols, seq, 1);
    return up256(frag_bytes(seq, cols)) + up256(partial_bytes(pl, seq, rows, 1));
}

// Workspace of the gated FFN: X fragments | H fragments | partial sums (the
// larger stage's; the stages run in order).
int64_t mm_ffn_workspace(int64_t seq, int64_t hidden, int64_t inter)
{
    const MmPlan pg = plan_of(inter, hidden, seq, 2), pd = plan_of(hidden, inter, seq, 1);
    const int64_t pa = partial_bytes(pg, seq, inter, 2), pb = partial_bytes(pd, seq, hidden, 1);
    return up256(frag_bytes(seq, hidden)) + up256(frag_bytes(seq, inter)) + up256(pa > pb ? pa : pb);
}

hipError_t launch_matmul_mfma(const uint8_t *W, const float *X, float *Y, int64_t rows,
                              int64_t cols, int64_t seq, uint8_t *ws, hipStream_t s)
{
    const MmPlan pl = plan_of(rows, cols, seq, 1);
    uint8_t *Xf = ws;
    float *partial = (float *)(Xf + up256(frag_bytes(seq, cols)));
    hipError_t e = launch_x_to_frag(X, Xf, seq, cols, s);
    if (e != hipSuccess) return e;
    MmArgs a{};
    a.W0 = W;
    a.W1 = W;
    a.Xf = Xf;
    a.out = Y;
    a.partial = partial;
    a.rows = (int32_t)rows;
    a.nb = (int32_t)(cols / 256);
    a.seq = (int32_t)seq;
    a.n_tiles = pl.n_t;
    a.S = pl.S;
    a.kps = pl.kps;
    e = launch_mm<1>(a, pl, s);
    if (e != hipSuccess || pl.S == 1) return e;
    return launch_reduce_y(partial, Y, seq * rows, pl.S, s);
}

hipError_t launch_ffn_prefill_mfma(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd,
                                   const float *X, float *Y, int64_t seq, int64_t hidden,
                                   int64_t inter, int act, uint8_t *ws, hipStream_t s)
{
    const MmPlan pg = plan_of(inter, hidden, seq, 2), pd = plan_of(hidden, inter, seq, 1);
    uint8_t *Xf = ws;
    uint8_t *Hf = Xf + up256(frag_bytes(seq, hidden));
    float *partial = (float *)(Hf + up256(frag_bytes(seq, inter)));
    hipError_t e = launch_x_to_frag(X, Xf, seq, hidden, s);
    if (e != hipSuccess) return e;

    MmArgs a{};
    a.W0 = Wg;
    a.W1 = Wu;
    a.Xf = Xf;
    a.out = Hf;
    a.partial = partial;
    a.rows = (int32_t)inter;
    a.nb = (int32_t)(hidden / 256);
    a.seq = (int32_t)seq;
    a.n_tiles = pg.n_t;
    a.S = pg.S;
    a.kps = pg.kps;
    a.act = act;
    a.out_kb = (int32_t)(inter / 256);
    e = launch_mm<2>(a, pg, s);
    if (e != hipSuccess) return e;
    if (pg.S > 1) {
        const int64_t seq_pad = pg.tg * kTokGroup, n = seq_pad * inter;
        hipLaunchKernelGGL(reduce_gated_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           partial, Hf, seq, seq_pad, inter, pg.S, act);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    MmArgs d{};
    d.W0 = Wd;
    d.W1 = Wd;
    d.Xf = Hf;
    d.out = Y;
    d.partial = partial;
    d.rows = (int32_t)hidden;
    d.nb = (int32_t)(inter / 256);
    d.seq = (int32_t)seq;
    d.n_tiles = pd.n_t;
    d.S = pd.S;
    d.kps = pd.kps;
    e = launch_mm<1>(d, pd, s);
    if (e != hipSuccess || pd.S == 1) return e;
    return launch_reduce_y(partial, Y, seq * hidden, pd.S, s);
}

}  // namespace q4k
