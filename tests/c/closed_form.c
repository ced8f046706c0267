/* Drives the library through its C ABI alone (no Python, no PyTorch): device
 * memory from hipMalloc, the cache on a HIP stream of its own, and closed forms
 * of the method's attention checked on what comes back.
 *  - A window of one key: the softmax over a single score is 1, so every query
 *    head returns the value row of its KV head, bit for bit in bf16.
 *  - A zero query: every score is 0, so each head returns the mean of the
 *    window's value rows (to bf16 rounding), also once the window slides.
 *  - The per-stream state after 65 appends into a ring of 64 slots.
 * Exit status 0 on success; otherwise the number of the failed check. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "a8r.h"

enum { NB = 2, HQ = 16, HKV = 2, D = 128, W = 64, G = HQ / HKV };

static uint32_t lcg_state = 12345u;
static float uniform(void) {           /* in [-1, 1) */
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return (float)((lcg_state >> 8) & 0xffffff) / 8388608.0f - 1.0f;
}
static uint16_t to_bf16(float f) {     /* round to nearest even; finite input */
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

#define CHECK(cond, code)                                                              \
    do {                                                                               \
        if (!(cond)) {                                                                 \
            fprintf(stderr, "check %d failed: %s (%s)\n", code, #cond, a8r_last_error()); \
            return code;                                                               \
        }                                                                              \
    } while (0)

static uint16_t hist_v[W + 1][NB][HKV][D];   /* every appended value row */

int main(void) {
    hipStream_t s;
    CHECK(hipStreamCreate(&s) == hipSuccess, 1);
    a8r_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.n_layers = 1; cfg.n_streams = NB; cfg.n_q_heads = HQ; cfg.n_kv_heads = HKV;
    cfg.head_dim = D; cfg.window = W; cfg.max_chunk = 1; cfg.dtype = A8R_BF16;
    cfg.rope_theta = 1.0e6;
    a8r_cache* c = NULL;
    CHECK(a8r_cache_create(&cfg, (void*)s, NULL, 0, &c) == A8R_OK, 2);
    const int64_t start[NB] = {1000000007, 5};
    const int32_t slot0[NB] = {17, 0};
    CHECK(a8r_reset(c, 0, NB, start, slot0) == A8R_OK, 3);

    uint16_t hk[NB][HKV][D], hq[NB][HQ][D], ho[NB][HQ][D];
    void *dk, *dv, *dq, *dout;
    CHECK(hipMalloc(&dk, sizeof hk) == hipSuccess, 4);
    CHECK(hipMalloc(&dv, sizeof hk) == hipSuccess, 4);
    CHECK(hipMalloc(&dq, sizeof hq) == hipSuccess, 4);
    CHECK(hipMalloc(&dout, sizeof ho) == hipSuccess, 4);

    for (int t = 0; t <= W; ++t) {
        for (int b = 0; b < NB; ++b)
            for (int h = 0; h < HKV; ++h)
                for (int d = 0; d < D; ++d) {
                    hk[b][h][d] = to_bf16(uniform());
                    hist_v[t][b][h][d] = to_bf16(uniform());
                }
        const int zero_q = t > 0;
        for (int b = 0; b < NB; ++b)
            for (int h = 0; h < HQ; ++h)
                for (int d = 0; d < D; ++d) hq[b][h][d] = zero_q ? 0 : to_bf16(uniform());
        CHECK(hipMemcpy(dk, hk, sizeof hk, hipMemcpyHostToDevice) == hipSuccess, 5);
        CHECK(hipMemcpy(dv, hist_v[t], sizeof hk, hipMemcpyHostToDevice) == hipSuccess, 5);
        CHECK(hipMemcpy(dq, hq, sizeof hq, hipMemcpyHostToDevice) == hipSuccess, 5);
        if (t == W) {
            /* the window is full: the fused call evicts token 0 and attends */
            CHECK(a8r_append_decode_attn(c, 0, 0, NB, dk, dv, dq, dout, NULL, NULL) == A8R_OK, 6);
        } else {
            CHECK(a8r_append_kv(c, 0, 0, NB, 1, dk, dv, NULL, NULL) == A8R_OK, 6);
            if (t != 0 && t != W - 1) continue;
            CHECK(a8r_decode_attn(c, 0, 0, NB, dq, dout) == A8R_OK, 7);
        }
        CHECK(hipStreamSynchronize(s) == hipSuccess, 8);
        CHECK(hipMemcpy(ho, dout, sizeof ho, hipMemcpyDeviceToHost) == hipSuccess, 8);
        for (int b = 0; b < NB; ++b)
            for (int h = 0; h < HQ; ++h)
                for (int d = 0; d < D; ++d) {
                    if (t == 0) {
                        CHECK(ho[b][h][d] == hist_v[0][b][h / G][d], 10);
                    } else {
                        const int first = t == W ? 1 : 0;   /* oldest live token */
                        double mean = 0.0;
                        for (int j = first; j <= t; ++j) mean += from_bf16(hist_v[j][b][h / G][d]);
                        mean /= (double)(t - first + 1);
                        CHECK(fabs(from_bf16(ho[b][h][d]) - mean) <= 1.0 / 256.0 * fabs(mean) + 1e-4, 11);
                    }
                }
    }
    for (int b = 0; b < NB; ++b) {
        int64_t p;
        int32_t l, sl;
        CHECK(a8r_get_state(c, 0, b, &p, &l, &sl) == A8R_OK, 12);
        CHECK(p == start[b] + W + 1 && l == W && sl == (slot0[b] + W + 1) % W, 13);
    }
    a8r_cache_destroy(c);
    (void)hipFree(dk);
    (void)hipFree(dv);
    (void)hipFree(dq);
    (void)hipFree(dout);
    (void)hipStreamDestroy(s);
    printf("closed forms hold: %s\n", a8r_version());
    return 0;
}
