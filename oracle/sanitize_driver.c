/*
 * Sanitizer driver for the oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Built together with dcconv_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer by the CPU test suite, it calls every oracle entry
 * point on small deterministic inputs -- valid calls, edge shapes (empty
 * sequences, one token, L > W-1, strided layouts) and every refusal path -- so
 * that an out-of-bounds access or undefined behaviour anywhere in the oracle
 * aborts the run.  It checks no values (the pinning tests do that).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float f);
uint32_t oracle_bf16_to_f32_bits(uint16_t b);
uint16_t oracle_f32_bits_to_bf16(uint32_t bits);
int oracle_update(const uint16_t *x, int64_t n_rows, int64_t d, int64_t ld, uint16_t *state, int64_t s_slots,
                  int64_t l, int64_t st_s, int64_t st_d, int64_t st_l, const uint16_t *weight, int64_t w,
                  const uint16_t *bias, const int32_t *indices, int activation, uint16_t *out, float *out_f32);
int oracle_update_tokens(const uint16_t *x, int64_t n_rows, int64_t d, int64_t t_steps, int64_t xs_n, int64_t xs_d,
                         int64_t xs_t, uint16_t *state, int64_t s_slots, int64_t l, int64_t st_s, int64_t st_d,
                         int64_t st_l, const uint16_t *weight, int64_t w, const uint16_t *bias,
                         const int32_t *indices, int activation, uint16_t *out, float *out_f32, int64_t os_n,
                         int64_t os_d, int64_t os_t);
int oracle_prefill(const uint16_t *x, int64_t n_seqs, int64_t d, int64_t t, int64_t xs_n, int64_t xs_d, int64_t xs_t,
                   const int32_t *starts, uint16_t *state, int64_t s_slots, int64_t l, int64_t st_s, int64_t st_d,
                   int64_t st_l, const int32_t *indices, const uint8_t *has_init, const uint16_t *weight, int64_t w,
                   const uint16_t *bias, int activation, uint16_t *out, float *out_f32, int64_t os_n, int64_t os_d,
                   int64_t os_t);
int oracle_update_ring(const uint16_t *x, int64_t n_rows, int64_t d, int64_t ld, uint16_t *state, int64_t s_slots,
                       int64_t l, int64_t st_s, int64_t st_d, int64_t st_l, const uint16_t *weight, int64_t w,
                       const uint16_t *bias, const int32_t *indices, const int32_t *cache_seqlens, int activation,
                       uint16_t *out, float *out_f32);

static uint32_t rng_state = 12345u;
static uint16_t rnd_bf16(void) {  /* a finite BF16 in about [-4, 4] */
    rng_state = rng_state * 1664525u + 1013904223u;
    uint16_t exp = (uint16_t)(120 + (rng_state >> 28) % 10);
    return (uint16_t)(((rng_state >> 8) & 0x8000u) | (exp << 7) | ((rng_state >> 12) & 0x7fu));
}
static uint16_t *bf_buf(size_t n) {  /* exactly n elements, so ASan sees any overrun */
    uint16_t *p = (uint16_t *)malloc((n ? n : 1) * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) p[i] = rnd_bf16();
    return p;
}

static int expect(int got, int want, const char *what) {
    if (got != want) {
        fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
        return 1;
    }
    return 0;
}

int main(void) {
    int bad = 0;
    /* conversions at the edges */
    const float vals[] = {0.0f, -0.0f, 1e-45f, 3.4e38f, -3.4e38f, 1.0f / 0.0f};
    for (int i = 0; i < 6; ++i) (void)oracle_bf16_to_f32(oracle_f32_to_bf16(vals[i]));
    for (uint32_t b = 0; b < 65536u; b += 97u) (void)oracle_f32_to_bf16(oracle_bf16_to_f32((uint16_t)b));
    for (uint32_t b = 0; b < 65536u; b += 97u)
        (void)oracle_f32_bits_to_bf16(oracle_bf16_to_f32_bits((uint16_t)b) | 1u);

    for (int64_t l = 3; l <= 9; l += 3) {
        const int64_t n = 5, d = 7, s = 8, w = 4, t = 6, ld = 9;
        uint16_t *x = bf_buf((size_t)(n * ld)), *weight = bf_buf((size_t)(d * w)), *bias = bf_buf((size_t)d);
        uint16_t *state = bf_buf((size_t)(s * d * l)), *out = bf_buf((size_t)(n * d));
        float *out32 = (float *)malloc((size_t)(n * d) * sizeof(float));
        int32_t idx[5] = {3, -1, 0, 7, -1};
        /* one step: compact and channel-last */
        bad += expect(oracle_update(x, n, d, ld, state, s, l, d * l, l, 1, weight, w, bias, idx, 1, out, out32), 0,
                      "update compact");
        bad += expect(oracle_update(x, n, d, ld, state, s, l, l * d, 1, d, weight, w, NULL, NULL, 0, out, NULL), 0,
                      "update channel-last");
        /* refusals */
        int32_t dup[5] = {1, 1, -1, -1, -1}, oob[5] = {0, 8, -1, -1, -1};
        bad += expect(oracle_update(x, n, d, ld, state, s, l, d * l, l, 1, weight, w, bias, dup, 0, out, NULL), 3, "dup");
        bad += expect(oracle_update(x, n, d, ld, state, s, l, d * l, l, 1, weight, w, bias, oob, 0, out, NULL), 2, "oob");
        bad += expect(oracle_update(x, n, d, d - 1, state, s, l, d * l, l, 1, weight, w, bias, idx, 0, out, NULL), 1,
                      "ld < d");
        /* multi-token: token-major and channel-major x */
        uint16_t *xt = bf_buf((size_t)(n * t * d)), *ot = bf_buf((size_t)(n * t * d));
        float *ot32 = (float *)malloc((size_t)(n * t * d) * sizeof(float));
        bad += expect(oracle_update_tokens(xt, n, d, t, t * d, 1, d, state, s, l, d * l, l, 1, weight, w, bias, idx, 1,
                                           ot, ot32, t * d, 1, d), 0, "tokens token-major");
        bad += expect(oracle_update_tokens(xt, n, d, t, d * t, t, 1, state, s, l, d * l, l, 1, weight, w, NULL, NULL, 0,
                                           ot, NULL, d * t, t, 1), 0, "tokens channel-major");
        /* prefill: batch, packed with empty and short sequences, stateless */
        int32_t starts[6] = {0, 0, 1, 3, 3, 30};
        uint8_t hi[5] = {1, 0, 1, 1, 0};
        uint16_t *xp = bf_buf((size_t)(30 * d)), *op = bf_buf((size_t)(30 * d));
        bad += expect(oracle_prefill(xt, n, d, t, t * d, 1, d, NULL, state, s, l, d * l, l, 1, idx, hi, weight, w, bias,
                                     1, ot, ot32, t * d, 1, d), 0, "prefill batch");
        bad += expect(oracle_prefill(xp, 5, d, 30, 0, 1, d, starts, state, s, l, l * d, 1, d, NULL, hi, weight, w, NULL,
                                     0, op, NULL, 0, 1, d), 0, "prefill packed");
        bad += expect(oracle_prefill(xp, 5, d, 30, 0, 1, d, starts, NULL, 0, 0, 0, 0, 0, NULL, NULL, weight, w, bias, 1,
                                     op, NULL, 0, 1, d), 0, "prefill stateless");
        int32_t unordered[6] = {0, 5, 2, 3, 3, 30};
        bad += expect(oracle_prefill(xp, 5, d, 30, 0, 1, d, unordered, state, s, l, l * d, 1, d, NULL, hi, weight, w,
                                     NULL, 0, op, NULL, 0, 1, d), 1, "prefill unordered");
        /* ring */
        int32_t seen[5] = {0, 1, 2, 1000, 7}, neg[5] = {0, -1, 2, 3, 4};
        bad += expect(oracle_update_ring(x, n, d, ld, state, s, l, d * l, l, 1, weight, w, bias, idx, seen, 1, out, out32),
                      0, "ring");
        bad += expect(oracle_update_ring(x, n, d, ld, state, s, l, d * l, l, 1, weight, w, bias, idx, neg, 1, out, NULL),
                      1, "ring negative");
        free(x); free(weight); free(bias); free(state); free(out); free(out32);
        free(xt); free(ot); free(ot32); free(xp); free(op);
    }
    if (bad == 0) printf("sanitized oracle run: ok\n");
    return bad != 0;
}
