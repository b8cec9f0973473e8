/*
 * q4k_oracle.c -- plain, slow, single-threaded CPU reference for the Q4_K
 * decode path. TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the product library never does, and the
 * two share no code (this file includes nothing from the HIP library).
 *
 * Everything is computed in double precision from the exact input bytes and
 * f32 activations. Each dequantised weight d*sc*q - dmin*m is exact in double
 * (f16 values carry 11 significant bits, sc*q at most 10 bits, and the f16
 * exponent range spans < 53 bits), every product with an f32 activation is
 * exact, and the only rounding is the sequential double summation.
 *
 * Sources (the pages):
 *  - infer-compute README, "Shaders" table (Q4_K/Q6_K and Q4_K fused FFN rows):
 *    a Q4_K matrix-vector product, fused QKV projection, fused gate+up with a
 *    GEGLU (GELU-tanh or SiLU gate) feeding the down projection.
 *  - infer-compute README, "Quick Start" (q4k_matvec(data, x, rows, hidden)),
 *    "Design Principles" item 8 (Q4_K matches the GGUF/Ollama quantisation).
 *  - Performance -- infer-inference, "Activation Function Support" table
 *    (gated GELU-tanh for Gemma, gated SiLU for Llama-family models).
 *  - infer-inference README, Overview example (top-5 predictions from logits);
 *    Performance -- infer-inference, "Honest Path Breakdown" (lm_head on GPU).
 *  The byte layout itself is the public GGUF Q4_K super-block (the pages only
 *  assert compatibility with it): see q4o_dequant_block.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *  - the min term is subtracted: w = d*sc*q - dmin*m;
 *  - GEGLU applies the activation to the gate: h = act(gate) * up;
 *  - GELU-tanh is 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)));
 *  - top-k order is value descending then index ascending, NaN ranks last;
 *  - top-k probabilities are the plain softmax over all rows' logits (no
 *    temperature or soft-capping), and a NaN logit makes them all NaN;
 *  - prefill is the decode definition applied per token, exactly (no bf16);
 *    q4o_ffn_prefill_bf16 additionally models bf16 operand rounding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define Q4O_QK 256
#define Q4O_BLOCK 144

/* IEEE 754 binary16 -> double, from the format definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 = zero/subnormal,
 * exponent 31 = infinity/NaN. */
double q4o_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* frac/1024 * 2^-14 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);  /* (1+frac/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* The 12 scale bytes hold eight 6-bit scales and eight 6-bit mins.
 * Sub-blocks 0..3 keep theirs in the low 6 bits of bytes 0..3 (scales) and
 * 4..7 (mins). Sub-blocks 4..7 take their low 4 bits from bytes 8..11 (low
 * nibble = scale, high nibble = min) and their top 2 bits from the spare top
 * 2 bits of bytes 0..3 (scales) and 4..7 (mins). */
void q4o_unpack_scales(const uint8_t *s, int *sc, int *mn)
{
    for (int j = 0; j < 4; ++j) {
        sc[j] = s[j] & 63;
        mn[j] = s[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        sc[j] = (s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4);
        mn[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* The quant of element e (0..255) of a block. The 128 quant bytes form four
 * 32-byte groups; group g holds elements 64g..64g+31 in its low nibbles and
 * elements 64g+32..64g+63 in its high nibbles. */
static int q4o_quant(const uint8_t *qs, int e)
{
    const int g = e / 64, r = e % 64;
    return r < 32 ? (qs[32 * g + r] & 0x0f) : (qs[32 * g + r - 32] >> 4);
}

/* Dequantise one 144-byte block: w[e] = d * sc[s] * q[e] - dmin * m[s],
 * s = e / 32 the sub-block of element e. */
void q4o_dequant_block(const uint8_t *blk, double *w)
{
    int sc[8], mn[8];
    const double d = q4o_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
    const double dmin = q4o_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
    q4o_unpack_scales(blk + 4, sc, mn);
    for (int e = 0; e < Q4O_QK; ++e) {
        const int s = e / 32;
        w[e] = d * sc[s] * q4o_quant(blk + 16, e) - dmin * mn[s];
    }
}

/* Dense f64 copy of a rows x cols Q4_K matrix (row-major). */
void q4o_dequant(const uint8_t *W, int64_t rows, int64_t cols, double *out)
{
    const int64_t nb = cols / Q4O_QK;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t b = 0; b < nb; ++b)
            q4o_dequant_block(W + (i * nb + b) * Q4O_BLOCK, out + i * cols + b * Q4O_QK);
}

/* y_i = sum_j w_ij x_j and the tolerance scale A_i = sum_j |w_ij x_j|,
 * x given in double. Either output may be NULL. */
void q4o_matvec_f64(const uint8_t *W, const double *x, int64_t rows, int64_t cols,
                    double *y, double *A)
{
    const int64_t nb = cols / Q4O_QK;
    double w[Q4O_QK];
    for (int64_t i = 0; i < rows; ++i) {
        double acc = 0.0, mag = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            q4o_dequant_block(W + (i * nb + b) * Q4O_BLOCK, w);
            for (int e = 0; e < Q4O_QK; ++e) {
                const double t = w[e] * x[b * Q4O_QK + e];
                acc += t;
                mag += fabs(t);
            }
        }
        if (y) y[i] = acc;
        if (A) A[i] = mag;
    }
}

/* Same with an f32 activation vector (widened exactly to double). */
void q4o_matvec(const uint8_t *W, const float *x, int64_t rows, int64_t cols,
                double *y, double *A)
{
    double *xd = (double *)malloc((size_t)cols * sizeof(double));
    for (int64_t j = 0; j < cols; ++j) xd[j] = (double)x[j];
    q4o_matvec_f64(W, xd, rows, cols, y, A);
    free(xd);
}

/* GELU, tanh approximation. */
double q4o_gelu_tanh(double z)
{
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/* SiLU: z * sigmoid(z). */
double q4o_silu(double z)
{
    return z / (1.0 + exp(-z));
}

void q4o_act_array(const double *z, int64_t n, int act, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = act == 0 ? q4o_gelu_tanh(z[i]) : q4o_silu(z[i]);
}

/* Gated FFN for one activation vector:
 *   g = Wg x, u = Wu x (Wg, Wu: inter x hidden), h = act(g) * u,
 *   y = Wd h (Wd: hidden x inter), A = sum_j |wd_ij h_j| with this h.
 * act: 0 = GELU-tanh, 1 = SiLU. g, u, h, A may be NULL. */
void q4o_ffn_f64(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const double *x,
                 int64_t hidden, int64_t inter, int act,
                 double *y, double *A, double *g_out, double *u_out, double *h_out)
{
    double *g = (double *)malloc((size_t)inter * sizeof(double));
    double *u = (double *)malloc((size_t)inter * sizeof(double));
    double *h = (double *)malloc((size_t)inter * sizeof(double));
    q4o_matvec_f64(Wg, x, inter, hidden, g, NULL);
    q4o_matvec_f64(Wu, x, inter, hidden, u, NULL);
    for (int64_t i = 0; i < inter; ++i)
        h[i] = (act == 0 ? q4o_gelu_tanh(g[i]) : q4o_silu(g[i])) * u[i];
    q4o_matvec_f64(Wd, h, hidden, inter, y, A);
    if (g_out) memcpy(g_out, g, (size_t)inter * sizeof(double));
    if (u_out) memcpy(u_out, u, (size_t)inter * sizeof(double));
    if (h_out) memcpy(h_out, h, (size_t)inter * sizeof(double));
    free(g);
    free(u);
    free(h);
}

/* The same with an f32 activation vector (widened exactly). */
void q4o_ffn(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const float *x,
             int64_t hidden, int64_t inter, int act,
             double *y, double *A, double *g_out, double *u_out, double *h_out)
{
    double *xd = (double *)malloc((size_t)hidden * sizeof(double));
    for (int64_t j = 0; j < hidden; ++j) xd[j] = (double)x[j];
    q4o_ffn_f64(Wg, Wu, Wd, xd, hidden, inter, act, y, A, g_out, u_out, h_out);
    free(xd);
}

/* ---- RMSNorm of the residual stream, the step before a projection ----
 * Sources: infer-compute README, "Key Optimizations" table (cooperative
 * rms_norm / residual_norm) and "Shaders" table (fused residual_norm);
 * Performance -- infer-inference, "Norm comparison" table (RMSNorm).
 * The residual stream is f32: s = h + delta is one IEEE single addition
 * (delta may be NULL: s = h). Then, in double,
 *   x_j = s_j / sqrt(mean_k(s_k^2) + eps) * w_j,
 * w the norm's weight vector (a model whose norm scales by 1 + w passes
 * 1 + w). s_out (f32) and x_out (f64) receive s and x. */
void q4o_residual_rmsnorm(const float *h, const float *delta, const float *w, float eps,
                          int64_t n, float *s_out, double *x_out)
{
    double ss = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const float a = h[j], b = delta ? delta[j] : 0.0f;
        const float sj = delta ? a + b : a;   /* one f32 rounding */
        s_out[j] = sj;
        ss += (double)sj * (double)sj;
    }
    const double inv = 1.0 / sqrt(ss / (double)n + (double)eps);
    for (int64_t j = 0; j < n; ++j) x_out[j] = (double)s_out[j] * inv * (double)w[j];
}

/* Derivatives of the activations, written from their definitions:
 * gelu_tanh(z) = 0.5 z (1 + t), t = tanh(c (z + 0.044715 z^3)), c = sqrt(2/pi):
 *   d/dz = 0.5 (1 + t) + 0.5 z (1 - t^2) c (1 + 3 * 0.044715 z^2);
 * silu(z) = z s, s = 1 / (1 + e^-z):  d/dz = s (1 + z (1 - s)). */
double q4o_act_deriv(double z, int act)
{
    if (act == 0) {
        const double c = sqrt(2.0 / M_PI);
        const double t = tanh(c * (z + 0.044715 * z * z * z));
        return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * z * z);
    }
    const double s = 1.0 / (1.0 + exp(-z));
    return s * (1.0 + z * (1.0 - s));
}

/* Error scale of the gated FFN under relative rounding of its operands. With
 * A_g = sum_k |wg_jk x_k| and A_u likewise, a relative change of at most e in
 * every x, wg, wu and wd, and in h, moves y_i by at most, to first order,
 *   e * sum_j |wd_ij| (|act'(g_j) u_j| A_g,j + |act(g_j)| A_u,j + 2 |h_j|)
 * (the last term counts wd's and h's own rounding). Ap returns that factor of
 * e per token and output, [seq][hidden]; it is the tolerance scale of the
 * reduced-precision FFN, and it is never below the plain A of the last stage. */
void q4o_ffn_prefill_scale(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd,
                           const float *X, int64_t seq, int64_t hidden, int64_t inter, int act,
                           double *Ap)
{
    double *g = (double *)malloc((size_t)inter * sizeof(double));
    double *u = (double *)malloc((size_t)inter * sizeof(double));
    double *ag = (double *)malloc((size_t)inter * sizeof(double));
    double *au = (double *)malloc((size_t)inter * sizeof(double));
    double *m = (double *)malloc((size_t)inter * sizeof(double));
    double *wd = (double *)malloc((size_t)inter * sizeof(double));
    for (int64_t t = 0; t < seq; ++t) {
        const float *x = X + t * hidden;
        q4o_matvec(Wg, x, inter, hidden, g, ag);
        q4o_matvec(Wu, x, inter, hidden, u, au);
        for (int64_t j = 0; j < inter; ++j) {
            const double a = act == 0 ? q4o_gelu_tanh(g[j]) : q4o_silu(g[j]);
            m[j] = fabs(q4o_act_deriv(g[j], act) * u[j]) * ag[j] + fabs(a) * au[j] +
                   2.0 * fabs(a * u[j]);
        }
        for (int64_t i = 0; i < hidden; ++i) {
            q4o_dequant(Wd + i * (inter / 256) * 144, 1, inter, wd);
            double acc = 0.0;
            for (int64_t j = 0; j < inter; ++j) acc += fabs(wd[j]) * m[j];
            Ap[t * hidden + i] = acc;
        }
    }
    free(g);
    free(u);
    free(ag);
    free(au);
    free(m);
    free(wd);
}

/* ---- top-k: the first k entries of all rows ordered by (value descending,
 * index ascending); NaN values rank below every number, among themselves by
 * index. A full sort is the definition. ---- */
static const double *q4o_sort_vals;

static int q4o_rank_cmp(const void *pa, const void *pb)
{
    const int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    const double va = q4o_sort_vals[a], vb = q4o_sort_vals[b];
    const int na = isnan(va), nb = isnan(vb);
    if (na != nb) return na ? 1 : -1;
    if (!na && va != vb) return va > vb ? -1 : 1;
    return a < b ? -1 : (a > b ? 1 : 0);
}

void q4o_topk(const double *v, int64_t n, int k, int64_t *idx, double *val)
{
    int64_t *order = (int64_t *)malloc((size_t)n * sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) order[i] = i;
    q4o_sort_vals = v;
    qsort(order, (size_t)n, sizeof(int64_t), q4o_rank_cmp);
    for (int i = 0; i < k && i < n; ++i) {
        idx[i] = order[i];
        val[i] = v[order[i]];
    }
    free(order);
}

/* ---- Q6_K: the other K-quant (GGUF super-block, 210 bytes / 256 weights) ----
 * Sources: infer-compute README, "Shaders" table (q6k_matvec beside the Q4_K
 * kernels) and "Design Principles" item 8 (Q4_K and Q6_K match the GGUF /
 * Ollama quantisation). As for Q4_K the pages give no byte layout; it is the
 * public GGUF Q6_K block: ql[128] (low 4 bits of each quant), qh[64] (high 2
 * bits), scales[16] (signed 8-bit, one per 16 consecutive weights), then d
 * (binary16) in bytes 208-209. Weight e = 128n + 32j + l (half n, quarter
 * j, l = 0..31) has q = (nibble j/2 of ql[64n + 32(j%2) + l])
 *                     | ((qh[32n + l] >> 2j) & 3) << 4,
 * and w = d * scales[e/16] * (q - 32). Each w is exact in double (11 + 8 + 6
 * significant bits). */
#define Q6O_BLOCK 210

static int q6o_quant(const uint8_t *blk, int e)
{
    const int n = e / 128, j = (e % 128) / 32, l = e % 32;
    const uint8_t lo = blk[64 * n + 32 * (j % 2) + l];
    const int low = (j / 2) ? (lo >> 4) : (lo & 0x0f);
    const int high = (blk[128 + 32 * n + l] >> (2 * j)) & 3;
    return low | (high << 4);
}

void q6o_dequant_block(const uint8_t *blk, double *w)
{
    const double d = q4o_f16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
    for (int e = 0; e < Q4O_QK; ++e) {
        const int sc = (int8_t)blk[192 + e / 16];
        w[e] = d * sc * (q6o_quant(blk, e) - 32);
    }
}

void q6o_dequant(const uint8_t *W, int64_t rows, int64_t cols, double *out)
{
    const int64_t nb = cols / Q4O_QK;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t b = 0; b < nb; ++b)
            q6o_dequant_block(W + (i * nb + b) * Q6O_BLOCK, out + i * cols + b * Q4O_QK);
}

/* y_i = sum_j w_ij x_j and A_i = sum_j |w_ij x_j| for a Q6_K matrix (either
 * output may be NULL). */
void q6o_matvec(const uint8_t *W, const float *x, int64_t rows, int64_t cols, double *y,
                double *A)
{
    const int64_t nb = cols / Q4O_QK;
    double w[Q4O_QK];
    for (int64_t i = 0; i < rows; ++i) {
        double acc = 0.0, mag = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            q6o_dequant_block(W + (i * nb + b) * Q6O_BLOCK, w);
            for (int e = 0; e < Q4O_QK; ++e) {
                const double t = w[e] * (double)x[b * Q4O_QK + e];
                acc += t;
                mag += fabs(t);
            }
        }
        if (y) y[i] = acc;
        if (A) A[i] = mag;
    }
}

/* ---- softmax over all rows (the probability of a top-k prediction) ----
 * Source: infer-inference README, Overview example (the top prediction is
 * shown with its probability in percent); Performance -- infer-inference,
 * "Real vindex" table (top prediction with its probability).
 * lse = log sum_i exp(v_i); p_i = exp(v_i - lse). The largest value m is
 * taken out first, lse = m + log sum_i exp(v_i - m), an exact identity that
 * keeps every exp() in (0, 1]. NaN anywhere makes lse (and so every p) NaN:
 * NaN never wins the comparison for m, but exp(NaN - m) poisons the sum. */
double q4o_logsumexp(const double *v, int64_t n)
{
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
        if (v[i] > m) m = v[i];
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += exp(v[i] - m);
    return m + log(s);
}

void q4o_softmax(const double *v, int64_t n, double *p)
{
    const double lse = q4o_logsumexp(v, n);
    for (int64_t i = 0; i < n; ++i) p[i] = exp(v[i] - lse);
}

/* ---- prefill: the decode definitions applied to each token row ---- */

/* Y[t][i] = sum_j w_ij X[t][j], A[t][i] = sum_j |w_ij X[t][j]|. */
void q4o_matmul(const uint8_t *W, const float *X, int64_t seq, int64_t rows, int64_t cols,
                double *Y, double *A)
{
    for (int64_t t = 0; t < seq; ++t)
        q4o_matvec(W, X + t * cols, rows, cols, Y + t * rows, A ? A + t * rows : NULL);
}

/* Per-token gated FFN; Y, A are [seq][hidden]. */
void q4o_ffn_prefill(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const float *X,
                     int64_t seq, int64_t hidden, int64_t inter, int act, double *Y, double *A)
{
    for (int64_t t = 0; t < seq; ++t)
        q4o_ffn(Wg, Wu, Wd, X + t * hidden, hidden, inter, act,
                Y + t * hidden, A ? A + t * hidden : NULL, NULL, NULL, NULL);
}

/* ---- bf16 operand model for the matrix-core prefill ----
 * bf16 keeps the top 16 bits of an IEEE binary32 value; conversion rounds to
 * nearest, ties to even. Weights are first formed in binary32 (the exact weight
 * rounded once to nearest even), then rounded to bf16. */
static double q4o_round_f32(double v)
{
    return (double)(float)v;   /* C conversion double->float rounds to nearest even */
}

double q4o_round_bf16(double v)
{
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    const float f = (float)v;  /* binary32 first (exact for binary32 inputs) */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    const uint32_t lsb = (bits >> 16) & 1u;
    bits += 0x7fffu + lsb;     /* round to nearest even at bit 16 */
    bits &= 0xffff0000u;
    float r;
    memcpy(&r, &bits, sizeof r);
    return (double)r;
}

/* Matrix product with bf16 operands: X rounded to bf16, W formed in binary32
 * and rounded to bf16, products and sums exact (f64). A as in q4o_matmul but
 * from the bf16 operands. A tighter second check of the matrix-core path. */
void q4o_matmul_bf16(const uint8_t *W, const float *X, int64_t seq, int64_t rows, int64_t cols,
                     double *Y, double *A)
{
    double *w = (double *)malloc((size_t)cols * sizeof(double));
    double *xb = (double *)malloc((size_t)(seq * cols) * sizeof(double));
    for (int64_t i = 0; i < seq * cols; ++i) xb[i] = q4o_round_bf16((double)X[i]);
    for (int64_t i = 0; i < rows; ++i) {
        q4o_dequant(W + i * (cols / 256) * 144, 1, cols, w);
        for (int64_t j = 0; j < cols; ++j) w[j] = q4o_round_bf16(q4o_round_f32(w[j]));
        for (int64_t t = 0; t < seq; ++t) {
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < cols; ++j) {
                const double p = w[j] * xb[t * cols + j];
                acc += p;
                mag += fabs(p);
            }
            Y[t * rows + i] = acc;
            if (A) A[t * rows + i] = mag;
        }
    }
    free(w);
    free(xb);
}

/* Per-token gated FFN with bf16 operands: X and W rounded to bf16 (W via
 * binary32), G and U exact products of those, H = act(G)*U rounded to bf16,
 * Y = Wd(bf16) H(bf16) exact. Used as a tighter second check of the matrix-core
 * path; the graded comparison is against q4o_ffn_prefill. */
void q4o_ffn_prefill_bf16(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd,
                          const float *X, int64_t seq, int64_t hidden, int64_t inter,
                          int act, double *Y, double *A)
{
    double *wg = (double *)malloc((size_t)(inter * hidden) * sizeof(double));
    double *wu = (double *)malloc((size_t)(inter * hidden) * sizeof(double));
    double *wd = (double *)malloc((size_t)(hidden * inter) * sizeof(double));
    double *xb = (double *)malloc((size_t)hidden * sizeof(double));
    double *h = (double *)malloc((size_t)inter * sizeof(double));
    q4o_dequant(Wg, inter, hidden, wg);
    q4o_dequant(Wu, inter, hidden, wu);
    q4o_dequant(Wd, hidden, inter, wd);
    for (int64_t i = 0; i < inter * hidden; ++i) {
        wg[i] = q4o_round_bf16(q4o_round_f32(wg[i]));
        wu[i] = q4o_round_bf16(q4o_round_f32(wu[i]));
        wd[i] = q4o_round_bf16(q4o_round_f32(wd[i]));
    }
    for (int64_t t = 0; t < seq; ++t) {
        for (int64_t j = 0; j < hidden; ++j) xb[j] = q4o_round_bf16((double)X[t * hidden + j]);
        for (int64_t i = 0; i < inter; ++i) {
            double g = 0.0, u = 0.0;
            for (int64_t j = 0; j < hidden; ++j) {
                g += wg[i * hidden + j] * xb[j];
                u += wu[i * hidden + j] * xb[j];
            }
            h[i] = q4o_round_bf16((act == 0 ? q4o_gelu_tanh(g) : q4o_silu(g)) * u);
        }
        for (int64_t i = 0; i < hidden; ++i) {
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < inter; ++j) {
                const double p = wd[i * inter + j] * h[j];
                acc += p;
                mag += fabs(p);
            }
            Y[t * hidden + i] = acc;
            if (A) A[t * hidden + i] = mag;
        }
    }
    free(wg);
    free(wu);
    free(wd);
    free(xb);
    free(h);
}
