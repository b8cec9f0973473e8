/* Test driver: every entry point of the oracle (oracle/q4k_oracle.c) on small
 * random inputs, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitize.py). Any out-of-bounds access, leak or undefined
 * operation aborts with a report; the numbers themselves are checked by the
 * pin tests, here only that every output is written and finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double q4o_f16_to_f64(uint16_t h);
void q4o_unpack_scales(const uint8_t *s, int *sc, int *mn);
void q4o_dequant_block(const uint8_t *blk, double *w);
void q4o_dequant(const uint8_t *W, int64_t rows, int64_t cols, double *out);
void q4o_matvec_f64(const uint8_t *W, const double *x, int64_t rows, int64_t cols, double *y, double *A);
void q4o_matvec(const uint8_t *W, const float *x, int64_t rows, int64_t cols, double *y, double *A);
double q4o_gelu_tanh(double z);
double q4o_silu(double z);
void q4o_act_array(const double *z, int64_t n, int act, double *out);
void q4o_ffn_f64(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const double *x,
                 int64_t hidden, int64_t inter, int act, double *y, double *A, double *g_out,
                 double *u_out, double *h_out);
void q4o_ffn(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const float *x,
             int64_t hidden, int64_t inter, int act, double *y, double *A, double *g_out,
             double *u_out, double *h_out);
void q4o_residual_rmsnorm(const float *h, const float *delta, const float *w, float eps, int64_t n,
                          float *s_out, double *x_out);
double q4o_act_deriv(double z, int act);
void q4o_ffn_prefill_scale(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const float *X,
                           int64_t seq, int64_t hidden, int64_t inter, int act, double *Ap);
void q4o_topk(const double *v, int64_t n, int k, int64_t *idx, double *val);
void q6o_dequant_block(const uint8_t *blk, double *w);
void q6o_dequant(const uint8_t *W, int64_t rows, int64_t cols, double *out);
void q6o_matvec(const uint8_t *W, const float *x, int64_t rows, int64_t cols, double *y, double *A);
double q4o_logsumexp(const double *v, int64_t n);
void q4o_softmax(const double *v, int64_t n, double *p);
void q4o_matmul(const uint8_t *W, const float *X, int64_t seq, int64_t rows, int64_t cols, double *Y,
                double *A);
void q4o_ffn_prefill(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const float *X,
                     int64_t seq, int64_t hidden, int64_t inter, int act, double *Y, double *A);
double q4o_round_bf16(double v);
void q4o_matmul_bf16(const uint8_t *W, const float *X, int64_t seq, int64_t rows, int64_t cols,
                     double *Y, double *A);
void q4o_ffn_prefill_bf16(const uint8_t *Wg, const uint8_t *Wu, const uint8_t *Wd, const float *X,
                          int64_t seq, int64_t hidden, int64_t inter, int act, double *Y, double *A);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 32);
}

/* random blocks with d and dmin set to small finite binary16 values */
static uint8_t *blocks(int64_t rows, int64_t cols, int bytes_per_block, int d_at)
{
    const int64_t n = rows * (cols / 256);
    uint8_t *W = malloc((size_t)(n * bytes_per_block));
    for (int64_t i = 0; i < n * bytes_per_block; ++i) W[i] = (uint8_t)next_u32();
    for (int64_t b = 0; b < n; ++b) {
        uint8_t *blk = W + b * bytes_per_block;
        blk[d_at] = 0x00; blk[d_at + 1] = 0x10;          /* d = 2^-11 */
        if (bytes_per_block == 144) { blk[2] = 0x00; blk[3] = 0x0C; } /* dmin = 2^-12 */
    }
    return W;
}

static float *vec(int64_t n)
{
    float *x = malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) x[i] = (float)((int32_t)next_u32() >> 8) / 8388608.0f;
    return x;
}

static int bad = 0;
static void check(const char *what, const double *v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) {
            fprintf(stderr, "%s[%lld] not finite\n", what, (long long)i);
            bad = 1;
            return;
        }
}

int main(void)
{
    const int64_t rows = 7, cols = 512, hidden = 256, inter = 512, seq = 3;
    /* f16, scales, blocks */
    double acc = 0.0;
    for (uint32_t h = 0; h < 65536; ++h) {
        const double v = q4o_f16_to_f64((uint16_t)h);
        if (isfinite(v)) acc += fabs(v);
    }
    uint8_t s12[12];
    int sc[8], mn[8];
    for (int i = 0; i < 12; ++i) s12[i] = (uint8_t)next_u32();
    q4o_unpack_scales(s12, sc, mn);
    uint8_t *W = blocks(rows, cols, 144, 0);
    double *dense = malloc((size_t)(rows * cols) * sizeof(double));
    q4o_dequant_block(W, dense);
    q4o_dequant(W, rows, cols, dense);
    check("dequant", dense, rows * cols);
    /* matvec (f32 and f64 inputs) */
    float *x = vec(cols);
    double *xd = malloc((size_t)cols * sizeof(double));
    for (int64_t i = 0; i < cols; ++i) xd[i] = x[i];
    double y[7], A[7];
    q4o_matvec(W, x, rows, cols, y, A);
    check("matvec", y, rows);
    q4o_matvec_f64(W, xd, rows, cols, y, NULL);
    q4o_matvec_f64(W, xd, rows, cols, NULL, A);
    /* activations */
    double z[5] = {-3.0, -0.5, 0.0, 0.5, 3.0}, za[5];
    for (int act = 0; act < 2; ++act) {
        q4o_act_array(z, 5, act, za);
        check("act", za, 5);
        for (int i = 0; i < 5; ++i) acc += q4o_act_deriv(z[i], act);
    }
    acc += q4o_gelu_tanh(1.0) + q4o_silu(1.0);
    /* FFN, both precisions, all optional outputs */
    uint8_t *Wg = blocks(inter, hidden, 144, 0), *Wu = blocks(inter, hidden, 144, 0);
    uint8_t *Wd = blocks(hidden, inter, 144, 0);
    float *xf = vec(hidden);
    double *xh = malloc((size_t)hidden * sizeof(double));
    for (int64_t i = 0; i < hidden; ++i) xh[i] = xf[i];
    double *fy = malloc((size_t)hidden * sizeof(double)), *fA = malloc((size_t)hidden * sizeof(double));
    double *g = malloc((size_t)inter * sizeof(double)), *u = malloc((size_t)inter * sizeof(double));
    double *hh = malloc((size_t)inter * sizeof(double));
    for (int act = 0; act < 2; ++act) {
        q4o_ffn(Wg, Wu, Wd, xf, hidden, inter, act, fy, fA, g, u, hh);
        check("ffn", fy, hidden);
        q4o_ffn(Wg, Wu, Wd, xf, hidden, inter, act, fy, NULL, NULL, NULL, NULL);
        q4o_ffn_f64(Wg, Wu, Wd, xh, hidden, inter, act, fy, fA, g, u, hh);
        check("ffn_f64", fy, hidden);
    }
    /* residual RMSNorm, with and without delta */
    float *h = vec(hidden), *dl = vec(hidden), *w = vec(hidden);
    float *s_out = malloc((size_t)hidden * sizeof(float));
    q4o_residual_rmsnorm(h, dl, w, 1e-6f, hidden, s_out, xh);
    check("rmsnorm", xh, hidden);
    q4o_residual_rmsnorm(h, NULL, w, 1e-6f, hidden, s_out, xh);
    /* top-k with ties and NaN, softmax */
    double v[9] = {1.0, 3.0, NAN, 3.0, -INFINITY, 2.0, 0.0, -0.0, 5.0}, p[9], val[9];
    int64_t idx[9];
    for (int k = 1; k <= 9; ++k) q4o_topk(v, 9, k, idx, val);
    acc += q4o_logsumexp(v + 3, 6);
    q4o_softmax(v + 3, 6, p);
    check("softmax", p, 6);
    /* Q6_K */
    uint8_t *W6 = blocks(rows, cols, 210, 208);
    q6o_dequant_block(W6, dense);
    q6o_dequant(W6, rows, cols, dense);
    check("q6 dequant", dense, rows * cols);
    q6o_matvec(W6, x, rows, cols, y, A);
    check("q6 matvec", y, rows);
    /* prefill: exact, bf16 model, error scale */
    float *X = vec(seq * hidden);
    double *Y = malloc((size_t)(seq * inter) * sizeof(double)), *YA = malloc((size_t)(seq * inter) * sizeof(double));
    q4o_matmul(Wg, X, seq, inter, hidden, Y, YA);
    check("matmul", Y, seq * inter);
    q4o_matmul_bf16(Wg, X, seq, inter, hidden, Y, YA);
    check("matmul_bf16", Y, seq * inter);
    for (int act = 0; act < 2; ++act) {
        q4o_ffn_prefill(Wg, Wu, Wd, X, seq, hidden, inter, act, Y, YA);
        check("ffn_prefill", Y, seq * hidden);
        q4o_ffn_prefill_bf16(Wg, Wu, Wd, X, seq, hidden, inter, act, Y, YA);
        check("ffn_prefill_bf16", Y, seq * hidden);
        q4o_ffn_prefill_scale(Wg, Wu, Wd, X, seq, hidden, inter, act, YA);
        check("ffn_prefill_scale", YA, seq * hidden);
    }
    acc += q4o_round_bf16(1.0 / 3.0);
    free(W); free(dense); free(x); free(xd); free(Wg); free(Wu); free(Wd); free(xf); free(xh);
    free(fy); free(fA); free(g); free(u); free(hh); free(h); free(dl); free(w); free(s_out);
    free(W6); free(X); free(Y); free(YA);
    printf("oracle driver: %s (%g)\n", bad ? "non-finite output" : "ok", acc);
    return bad;
}
