/* Test driver: the argument checks of every libq4k entry point (include/q4k.h)
 * with the library's host code built under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitize.py). Every call here fails a
 * check (or is an empty no-op), so nothing is enqueued and no GPU is needed;
 * the buffers are host memory standing in for device pointers, never read. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "q4k.h"

static int fails = 0;
#define EXPECT(call, want)                                                          \
    do {                                                                            \
        const int got_ = (call);                                                    \
        if (got_ != (want)) {                                                       \
            fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, \
                    (want));                                                        \
            fails = 1;                                                              \
        }                                                                           \
    } while (0)

int main(void)
{
    const int64_t rows = 64, cols = 512, hidden = 256, inter = 512;
    uint8_t *arena = aligned_alloc(256, 1 << 22);
    uint8_t *W = arena;                         /* weights: 1 MiB */
    float *x = (float *)(arena + (1 << 20));    /* activations */
    float *y = (float *)(arena + (2 << 20));    /* outputs */
    float *z = (float *)(arena + (3 << 20));    /* more outputs / workspace */
    int32_t *ti = (int32_t *)(z + 1024);
    void *S = NULL;                             /* default stream (never used) */

    /* status strings */
    for (int s = 1; s >= -10; --s) {
        const char *m = q4k_status_string(s);
        if (!m || !m[0]) fails = 1;
    }
    (void)q4k_last_hip_error();

    /* matvec / q6k_matvec */
    EXPECT(q4k_matvec(W, x, y, rows, 100, S), Q4K_ERR_SHAPE);
    EXPECT(q4k_matvec(W, x, y, -1, cols, S), Q4K_ERR_SHAPE);
    EXPECT(q4k_matvec(W, x, y, rows, 65536 + 256, S), Q4K_ERR_SHAPE);
    EXPECT(q4k_matvec(W, x, y, 0, cols, S), Q4K_OK);
    EXPECT(q4k_matvec(NULL, x, y, rows, cols, S), Q4K_ERR_NULL);
    EXPECT(q4k_matvec(W + 1, x, y, rows, cols, S), Q4K_ERR_ALIGN);
    EXPECT(q4k_matvec(W, x, (float *)W, rows, cols, S), Q4K_ERR_ALIAS);
    EXPECT(q6k_matvec(W, x, y, rows, 100, S), Q4K_ERR_SHAPE);
    EXPECT(q6k_matvec(W, NULL, y, rows, cols, S), Q4K_ERR_NULL);
    EXPECT(q6k_matvec(W, x + 1, y, rows, cols, S), Q4K_ERR_ALIGN);
    /* qkv */
    EXPECT(q4k_qkv(W, x, y, y + 512, y + 1024, -1, 8, cols, S), Q4K_ERR_SHAPE);
    EXPECT(q4k_qkv(W, x, y, NULL, y + 1024, 16, 8, cols, S), Q4K_ERR_NULL);
    EXPECT(q4k_qkv(W, x, y, y + 8, y + 1024, 16, 8, cols, S), Q4K_ERR_ALIAS);
    EXPECT(q4k_qkv(W, x, y, y + 512, y + 1024, 0, 0, cols, S), Q4K_OK);
    /* gate_up / ffn */
    EXPECT(q4k_gate_up(W, W, x, y, inter, hidden, 7, S), Q4K_ERR_ACT);
    EXPECT(q4k_gate_up(W, NULL, x, y, inter, hidden, 0, S), Q4K_ERR_NULL);
    const size_t fws = q4k_ffn_workspace_bytes(hidden, inter);
    if (fws == 0) fails = 1;
    EXPECT(q4k_ffn(W, W, W, x, y, hidden, inter, 0, z, fws - 1, S), Q4K_ERR_WORKSPACE);
    EXPECT(q4k_ffn(W, W, W, x, y, hidden, inter, 2, z, fws, S), Q4K_ERR_ACT);
    EXPECT(q4k_ffn(W, W, W, x, y, hidden, 300, 0, z, fws, S), Q4K_ERR_SHAPE);
    /* fused norms */
    EXPECT(q4k_rmsnorm_matvec(W, x, NULL, x, -1.0f, NULL, y, rows, cols, S), Q4K_ERR_EPS);
    EXPECT(q4k_rmsnorm_matvec(W, x, NULL, NULL, 1e-6f, NULL, y, rows, cols, S), Q4K_ERR_NULL);
    EXPECT(q4k_rmsnorm_ffn(W, W, W, x, NULL, x, 1e-6f, NULL, y, hidden, inter, 0, z, fws - 1, S),
           Q4K_ERR_WORKSPACE);
    /* lm_head */
    const size_t lws = q4k_lmhead_workspace_bytes(rows, cols, 5);
    if (lws == 0) fails = 1;
    EXPECT(q4k_lmhead_topk(W, x, y, rows, cols, 0, ti, z, z + 64, lws, S), Q4K_ERR_K);
    EXPECT(q4k_lmhead_topk(W, x, y, rows, cols, 65, ti, z, z + 64, lws, S), Q4K_ERR_K);
    EXPECT(q4k_lmhead_topk(W, x, y, rows, cols, 5, ti, z, z + 64, lws - 1, S), Q4K_ERR_WORKSPACE);
    EXPECT(q4k_lmhead_topk_probs(W, x, y, rows, cols, 5, ti, z, NULL, z + 8, z + 64, lws, S),
           Q4K_ERR_NULL);
    /* the vocabulary limit */
    const int64_t rmax = q4k_lmhead_rows_max(cols);
    if (rmax < 4000000 || q4k_lmhead_workspace_bytes(rmax + 1, cols, 5) != 0) fails = 1;
    EXPECT(q4k_lmhead_topk(W, x, y, rmax + 1, cols, 5, ti, z, z + 64, (size_t)1 << 40, S),
           Q4K_ERR_SHAPE);
    /* measurement helpers */
    EXPECT(q4k_probe_read(W, 0, 256, 512, 8, 0, (uint32_t *)z, S), Q4K_ERR_SHAPE);
    EXPECT(q4k_probe_read(W, 4096, 256, 512, 3, 0, (uint32_t *)z, S), Q4K_ERR_SHAPE);
    EXPECT(q4k_probe_read(W, 4096, 256, 512, 8, 0, NULL, S), Q4K_ERR_NULL);
    EXPECT(q4k_probe_read(W, 4096, 256, 512, 8, 1, (uint32_t *)W, S), Q4K_ERR_ALIAS);
    EXPECT(q4k_probe_empty(0, 256, (uint32_t *)z, S), Q4K_ERR_SHAPE);
    /* prefill */
    EXPECT(q4k_matmul(W, x, y, rows, cols, -1, z, 0, S), Q4K_ERR_SHAPE);
    EXPECT(q4k_matmul(W, x, y, rows, cols, 0, z, 0, S), Q4K_OK);
    EXPECT(q4k_ffn_prefill(W, W, W, x, y, 4, hidden, inter, 9, z, 1 << 20, S), Q4K_ERR_ACT);
    EXPECT(q4k_ffn_prefill(W, W, W, NULL, y, 4, hidden, inter, 0, z, 1 << 20, S), Q4K_ERR_NULL);
    if (q4k_matmul_workspace_bytes(rows, cols, 64) == 0) fails = 1;
    if (q4k_ffn_prefill_workspace_bytes(64, hidden, inter) == 0) fails = 1;
    free(arena);
    printf("abi driver: %s\n", fails ? "FAILED" : "ok");
    return fails;
}
