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
// range of super-blocks (a K split), for 64 tokens. Four compute waves run in
// lockstep over the super-blocks:
//   * tiles 0..4A-1 are "own" tiles: wave w dequantises tiles wA..wA+A-1 into
//     its registers and multiplies them by all four token tiles;
//   * tiles 4A..4A+B-1 are "shared": all 256 compute threads dequantise them
//     into LDS (bf16), and wave w multiplies them by token tile w.
// Every wave then dequantises the same number of weights and issues the same
// number of MFMAs, whatever n_t is, so one workgroup per CU keeps all four
// SIMDs equally busy. A fifth wave only copies the activation fragments of
// the next super-blocks into an LDS ring with LDS-DMA loads; its wait counter
// is its own, so the compute waves' weight prefetch (a register ring of
// kRing - 1 super-blocks in flight) never waits on it.
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
typedef __attribute__((address_space(3))) void *lds_ptr;

constexpr int kTokGroup = 64;          // tokens per group (four 16-token tiles)
constexpr int kChunk = 32768;          // bytes of one super-block column of a token group
constexpr int kXBufs = 3;              // activation chunks in the LDS ring
constexpr int kRing = 5;               // weight register ring slots (4 blocks in flight)
constexpr int kComputeThreads = 256;
constexpr int kThreads = 320;          // + one loader wave
constexpr int kTileBytesPerBlock = 16 * kBlockBytes;

enum MmEpi { MM_EPI_Y = 0, MM_EPI_PARTIAL = 1, MM_EPI_GATED = 2 };

struct MmArgs {
    const uint8_t *W0;     // weights (gate matrix of the pair)
    const uint8_t *W1;     // up matrix of the pair (unused for one matrix)
    const uint8_t *Xf;     // bf16 activation fragments, KB = nb super-blocks per token group
    void *out;             // MM_EPI_Y: f32 [seq][rows]; MM_EPI_PARTIAL: f32 [S][seq][NMAT*rows];
                           // MM_EPI_GATED: bf16 fragments of H (KB = out_kb)
    int32_t rows;          // rows per matrix
    int32_t nb;            // super-blocks per weight row
    int32_t seq;
    int32_t n_tiles;       // tiles per workgroup (4A + B)
    int32_t S;             // K splits
    int32_t kps;           // super-blocks per split
    int32_t epi;
    int32_t act;
    int32_t out_kb;
};

__device__ __forceinline__ float act_apply(float z, int act)
{
    if (act == 0) {
        const float c = 0.7978845608028654f;  // sqrt(2/pi)
        return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
    }
    return z / (1.0f + expf(-z));
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

template <int A, int B>
struct WSlot {
    uint4 oh[A > 0 ? A : 1], oq0[A > 0 ? A : 1], oq1[A > 0 ? A : 1];   // own tiles: header, quants
    uint4 sh[B > 0 ? B : 1];                                          // shared tiles: header
    uint2 sq[B > 0 ? B : 1];                                          //   and 8 quant bytes
};

// LDS operands of one K-step: the four token tiles (own tiles), this wave's
// token tile and the shared tiles' weights.
template <int B>
struct Ops {
    bf16x8 xa[4], xw;
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

template <int NMAT, int A, int B>
__global__ __launch_bounds__(kThreads, 1) void mm_kernel(MmArgs p)
{
    __shared__ __attribute__((aligned(16))) uint8_t xbuf[kXBufs * kChunk];
    __shared__ __attribute__((aligned(16))) uint8_t bbuf[2 * (B > 0 ? B : 1) * 8 * 1024];

    const int rg = blockIdx.x / p.S, sp = blockIdx.x % p.S;
    const int64_t tg = blockIdx.y;
    const int kb0 = sp * p.kps;
    const int nblk = min(p.nb, kb0 + p.kps) - kb0;
    const int niter = (nblk + kRing - 1) / kRing * kRing;
    const int64_t tile0 = (int64_t)rg * p.n_tiles;
    const int t = threadIdx.x;
    const int wave = t >> 6, l = t & 63;

    if (wave == 4) {
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
        issue(0);
        if (nblk > 1) issue(1);
        for (int b = 0; b < niter; ++b) {
            if (b < nblk) wait_vmcnt_le(b + 1 < nblk ? 32 : 0);   // chunk b has landed
            barrier_lds();
            if (b + 2 < nblk) issue(b + 2);   // into the buffer chunk b-1 used
        }
        return;
    }

    const int n = l & 15, c = l >> 4;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int ns = t >> 4, q = t & 15;       // shared-tile dequant: row ns, quant piece q
    const uint8_t *rp_own[A > 0 ? A : 1];
    const uint8_t *rp_sh[B > 0 ? B : 1];
#pragma unroll
    for (int i = 0; i < A; ++i) rp_own[i] = row_ptr<NMAT>(p, tile0 + wave * A + i, n);
#pragma unroll
    for (int s = 0; s < B; ++s) rp_sh[s] = row_ptr<NMAT>(p, tile0 + 4 * A + s, ns);

    WSlot<A, B> ring[kRing];
    auto load = [&](WSlot<A, B> &sl, int b) {
        const int64_t off = (int64_t)(kb0 + min(b, nblk - 1)) * kBlockBytes;
#pragma unroll
        for (int i = 0; i < A; ++i) {
            const uint8_t *r = rp_own[i] + off;
            sl.oh[i] = *reinterpret_cast<const uint4 *>(r);
            sl.oq0[i] = *reinterpret_cast<const uint4 *>(r + 16 + 32 * c);
            sl.oq1[i] = *reinterpret_cast<const uint4 *>(r + 32 + 32 * c);
        }
#pragma unroll
        for (int s = 0; s < B; ++s) {
            const uint8_t *r = rp_sh[s] + off;
            sl.sh[s] = *reinterpret_cast<const uint4 *>(r);
            sl.sq[s] = *reinterpret_cast<const uint2 *>(r + 16 + 8 * q);
        }
    };
    // Shared tiles of one block -> LDS operand buffer `buf`.
    auto prep_shared = [&](const WSlot<A, B> &sl, int buf) {
#pragma unroll
        for (int s = 0; s < B; ++s) {
            const int g = q >> 2, jl = q & 3;
            const Coef k = block_coef(sl.sh[s], g);
            const bf16x8 lo = deq8<false>(sl.sq[s].x, sl.sq[s].y, k.a_lo, k.b_lo);
            const bf16x8 hi = deq8<true>(sl.sq[s].x, sl.sq[s].y, k.a_hi, k.b_hi);
            uint8_t *base = bbuf + (buf * B + s) * 8192;
            *reinterpret_cast<bf16x8 *>(base + (jl * 64 + b_pos(ns, g, jl)) * 16) = lo;
            *reinterpret_cast<bf16x8 *>(base + ((jl + 4) * 64 + b_pos(ns, g, jl + 4)) * 16) = hi;
        }
    };

    f32x4 acc[A > 0 ? A : 1][4];
    f32x4 acc_sh[B > 0 ? B : 1];
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[i][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < B; ++s) acc_sh[s] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int b = 0; b < kRing - 1; ++b) load(ring[b], b);
    // Keep all prologue loads ahead of the first wait (the scheduler would
    // otherwise issue blocks 1.. only after block 0 has arrived).
    asm volatile("" ::: "memory");
    if constexpr (B > 0) prep_shared(ring[0], 0);

    for (int b0 = 0; b0 < niter; b0 += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int b = b0 + u;
            barrier_lds();   // chunk b and the shared operands of block b are in LDS
            load(ring[(u + kRing - 1) % kRing], b + kRing - 1);
            if (b < nblk) {
                const uint8_t *xb = xbuf + (b % kXBufs) * kChunk;
                const WSlot<A, B> &sl = ring[u];
                Coef k[A > 0 ? A : 1];
#pragma unroll
                for (int i = 0; i < A; ++i) k[i] = block_coef(sl.oh[i], c);
                // LDS operands of K-step j+1 are requested before K-step j is
                // dequantised and multiplied, so their latency hides behind that work.
                const uint8_t *sbase = bbuf + ((b & 1) * B) * 8192;
                auto read_ops = [&](int j, Ops<B> &o) {
                    if constexpr (A > 0) {
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt)
                            o.xa[tt] = *reinterpret_cast<const bf16x8 *>(xb + ((j * 4 + tt) * 64 + l) * 16);
                    }
                    if constexpr (B > 0) {
                        // this wave's token tile, for the shared tiles (a second LDS
                        // read rather than a per-lane select or a branch)
                        o.xw = *reinterpret_cast<const bf16x8 *>(xb + ((j * 4 + wave_u) * 64 + l) * 16);
#pragma unroll
                        for (int s = 0; s < B; ++s)
                            o.wb[s] = *reinterpret_cast<const bf16x8 *>(sbase + s * 8192 + (j * 64 + b_pos(n, c, j)) * 16);
                    }
                };
                Ops<B> ops[2];
                read_ops(0, ops[0]);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (j + 1 < 8) read_ops(j + 1, ops[(j + 1) & 1]);
                    const Ops<B> &o = ops[j & 1];
#pragma unroll
                    for (int i = 0; i < A; ++i) {
                        const uint4 &qa = (j & 3) < 2 ? sl.oq0[i] : sl.oq1[i];
                        const uint32_t w0 = (j & 1) ? qa.z : qa.x, w1 = (j & 1) ? qa.w : qa.y;
                        const bf16x8 wb = j < 4 ? deq8<false>(w0, w1, k[i].a_lo, k[i].b_lo)
                                                : deq8<true>(w0, w1, k[i].a_hi, k[i].b_hi);
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt)
                            acc[i][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.xa[tt], wb, acc[i][tt], 0, 0, 0);
                    }
#pragma unroll
                    for (int s = 0; s < B; ++s)
                        acc_sh[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.xw, o.wb[s], acc_sh[s], 0, 0, 0);
                }
                if constexpr (B > 0) {
                    if (b + 1 < nblk) prep_shared(ring[(u + 1) % kRing], (b + 1) & 1);
                }
            }
        }
    }

    // ---- epilogue ----
    const int64_t tok_base = tg * kTokGroup;
    auto store = [&](f32x4 v, int64_t tile, int64_t tok0) {
        // lane (n, c), register r: token tok0 + 4c + r, tile row n
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t token = tok0 + 4 * c + r;
            const float val = v[r];
            if (p.epi == MM_EPI_GATED) {
                const float other = __int_as_float(
                    __builtin_amdgcn_update_dpp(0, __float_as_int(val), 0x128, 0xF, 0xF, false));
                const int64_t irow = 8 * tile + n;
                if (n < 8 && irow < p.rows) {
                    const float h = act_apply(val, p.act) * other;
                    *reinterpret_cast<__bf16 *>((uint8_t *)p.out + frag_offset(token, irow, p.out_kb)) = (__bf16)h;
                }
            } else if (token < p.seq) {
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
                float *o = (float *)p.out;
                if (p.epi == MM_EPI_PARTIAL) o += (int64_t)sp * p.seq * ncols;
                o[token * ncols + col] = val;
            }
        }
    };
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) store(acc[i][tt], tile0 + wave * A + i, tok_base + 16 * tt);
#pragma unroll
    for (int s = 0; s < B; ++s) store(acc_sh[s], tile0 + 4 * A + s, tok_base + 16 * wave);
}

// f32 activations [seq][cols] -> bf16 fragments (zeros for padding tokens).
__global__ __launch_bounds__(256) void x_to_frag_kernel(const float *X, uint8_t *Xf, int64_t seq,
                                                         int64_t cols, int64_t pieces)
{
    const int64_t pc = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (pc >= pieces) return;
    const int64_t KB = cols >> 8;
    const int lane = (int)pc & 63, tt = (int)(pc >> 6) & 3, j = (int)(pc >> 8) & 7;
    const int64_t rest = pc >> 11, kb = rest % KB, tg = rest / KB;
    const int64_t token = tg * kTokGroup + 16 * tt + (lane & 15);
    const int c = lane >> 4;
    const int64_t k0 = kb * 256 + 64 * c + 32 * (j >> 2) + 8 * (j & 3);
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
    *reinterpret_cast<bf16x8 *>(Xf + pc * 16) = v;
}

// Y[t][i] = sum_s P[s][t][i], s in order.
__global__ __launch_bounds__(256) void reduce_y_kernel(const float *P, float *Y, int64_t n, int S)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = P[i];
    for (int s = 1; s < S; ++s) acc += P[(int64_t)s * n + i];
    Y[i] = acc;
}

// Gate/up partials P[s][t][0..2 inter) -> H = act(G) * U as bf16 fragments
// for all tokens of the padded groups (zeros past seq).
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
        for (int s = 1; s < S; ++s) {
            g += pg[s * stride];
            u += pg[s * stride + inter];
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

constexpr int kMaxTilesPerWg = 8;

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
        double cost = (double)rounds * (double)n_t * kps * kTileBytesPerBlock * cus;
        if (S > 1) cost += 0.35 * (double)S * (double)seq * (double)rows_out * 8.0;
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
    const int64_t TG = (seq + kTokGroup - 1) / kTokGroup;
    const int64_t pieces = TG * (cols / 256) * 2048;
    hipLaunchKernelGGL(x_to_frag_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s,
                       X, Xf, seq, cols, pieces);
    return hipGetLastError();
}

}  // namespace

MmPlan mm_plan(int64_t rows, int64_t cols, int64_t seq, int nmat)
{
    const int64_t T = nmat == 1 ? (rows + 15) / 16 : (rows + 7) / 8;
    return plan_for(T, (int)(cols / 256), seq, rows * nmat, device_cus_mm());
}

int64_t mm_frag_bytes(int64_t seq, int64_t cols)
{
    return (seq + kTokGroup - 1) / kTokGroup * kTokGroup * cols * 2;
}

int64_t mm_partial_bytes(const MmPlan &pl, int64_t seq, int64_t rows, int nmat)
{
    return pl.S > 1 ? (int64_t)pl.S * seq * rows * nmat * 4 : 0;
}

hipError_t launch_matmul_mfma(const uint8_t *W, const float *X, float *Y, int64_t rows,
                              int64_t cols, int64_t seq, uint8_t *Xf, float *partial,
                              hipStream_t s)
{
    const MmPlan pl = mm_plan(rows, cols, seq, 1);
    hipError_t e = launch_x_to_frag(X, Xf, seq, cols, s);
    if (e != hipSuccess) return e;
    MmArgs a{};
    a.W0 = W;
    a.W1 = W;
    a.Xf = Xf;
    a.rows = (int32_t)rows;
    a.nb = (int32_t)(cols / 256);
    a.seq = (int32_t)seq;
    a.n_tiles = pl.n_t;
    a.S = pl.S;
    a.kps = pl.kps;
    a.epi = pl.S > 1 ? MM_EPI_PARTIAL : MM_EPI_Y;
    a.out = pl.S > 1 ? (void *)partial : (void *)Y;
    e = launch_mm<1>(a, pl, s);
    if (e != hipSuccess || pl.S == 1) return e;
    const int64_t nout = seq * rows;
    hipLaunchKernelGGL(reduce_y_kernel, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, s,
                       partial, Y, nout, pl.S);
    return hipGetLastError();
}

hipError_t launch_ffn_prefill_mfma(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd,
                                   const float *X, float *Y, int64_t seq, int64_t hidden,
                                   int64_t inter, int act, uint8_t *Xf, uint8_t *Hf,
                                   float *partial, hipStream_t s)
{
    const MmPlan pg = mm_plan(inter, hidden, seq, 2);
    const MmPlan pd = mm_plan(hidden, inter, seq, 1);
    hipError_t e = launch_x_to_frag(X, Xf, seq, hidden, s);
    if (e != hipSuccess) return e;

    MmArgs a{};
    a.W0 = Wg;
    a.W1 = Wu;
    a.Xf = Xf;
    a.rows = (int32_t)inter;
    a.nb = (int32_t)(hidden / 256);
    a.seq = (int32_t)seq;
    a.n_tiles = pg.n_t;
    a.S = pg.S;
    a.kps = pg.kps;
    a.act = act;
    a.out_kb = (int32_t)(inter / 256);
    a.epi = pg.S > 1 ? MM_EPI_PARTIAL : MM_EPI_GATED;
    a.out = pg.S > 1 ? (void *)partial : (void *)Hf;
    e = launch_mm<2>(a, pg, s);
    if (e != hipSuccess) return e;
    if (pg.S > 1) {
        const int64_t seq_pad = pg.tg * kTokGroup;
        const int64_t n = seq_pad * inter;
        hipLaunchKernelGGL(reduce_gated_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           partial, Hf, seq, seq_pad, inter, pg.S, act);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    MmArgs d{};
    d.W0 = Wd;
    d.W1 = Wd;
    d.Xf = Hf;
    d.rows = (int32_t)hidden;
    d.nb = (int32_t)(inter / 256);
    d.seq = (int32_t)seq;
    d.n_tiles = pd.n_t;
    d.S = pd.S;
    d.kps = pd.kps;
    d.epi = pd.S > 1 ? MM_EPI_PARTIAL : MM_EPI_Y;
    d.out = pd.S > 1 ? (void *)partial : (void *)Y;
    e = launch_mm<1>(d, pd, s);
    if (e != hipSuccess || pd.S == 1) return e;
    const int64_t nout = seq * hidden;
    hipLaunchKernelGGL(reduce_y_kernel, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0, s,
                       partial, Y, nout, pd.S);
    return hipGetLastError();
}

}  // namespace q4k
