/* Runs every function of the CPU oracle on small, degenerate and ragged inputs
 * under AddressSanitizer and UndefinedBehaviorSanitizer (built and run by
 * tests/test_sanitizers.py). Exit status 0 means every run completed and every
 * checked value matched; a sanitizer report aborts with a non-zero status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_absmean(const float *w, int64_t n, int64_t k);
void oracle_ternarize(const float *w, int64_t n, int64_t k, float gamma, int8_t *wt);
float oracle_threshold_ternarize(const float *w, int64_t n, int64_t k, float factor, int8_t *wt, float *delta);
void oracle_pack(const int8_t *wt, int64_t n, int64_t k, uint8_t *packed);
void oracle_pack_kmajor(const uint8_t *packed, int64_t n, int64_t k, uint8_t *out);
int64_t oracle_unpack(const uint8_t *packed, int64_t n, int64_t k, int8_t *wt);
void oracle_quant_act(const float *x, int64_t m, int64_t k, int8_t *q, float *s);
void oracle_quant_act_a4(const float *x, int64_t m, int64_t k, int64_t keep, int8_t *q, float *s);
int oracle_e2m1_doubled(float v);
void oracle_matmul_i32(const int8_t *q, int64_t m, int64_t k, const int8_t *wt, int64_t n, int32_t *acc);
void oracle_rescale(const int32_t *acc, int64_t m, int64_t n, const float *s, float gamma, float *y);
void oracle_rescale_q(const int32_t *acc, int64_t m, int64_t n, const float *s, float gamma, float qmax, float *y);
void oracle_sqrelu_gate(const float *g, const float *u, int64_t count, float *h);
void oracle_bf16_to_f32(const uint16_t *x, int64_t count, float *out);

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++failures; } } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static float frand(void)  /* xorshift64*, uniform in [-1, 1) */
{
    state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
    return (float)((double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static void run_linear(int64_t m, int64_t k, int64_t n, float scale_w, int zero_token)
{
    float *w = malloc(sizeof(float) * n * k), *x = malloc(sizeof(float) * m * k);
    int8_t *wt = malloc(n * k), *wt2 = malloc(n * k), *q = malloc(m * k);
    uint8_t *p = malloc(n * k / 4), *pt = malloc(n * k / 4 + 1);
    int32_t *acc = malloc(sizeof(int32_t) * m * n);
    float *s = malloc(sizeof(float) * m), *y = malloc(sizeof(float) * m * n), delta;
    for (int64_t i = 0; i < n * k; ++i) w[i] = scale_w * frand();
    for (int64_t i = 0; i < m * k; ++i) x[i] = 4.0f * frand();
    if (zero_token) memset(x, 0, sizeof(float) * k);
    const float g = oracle_absmean(w, n, k);
    oracle_ternarize(w, n, k, g, wt);
    oracle_pack(wt, n, k, p);
    CHECK(oracle_unpack(p, n, k, wt2) == 0);
    CHECK(memcmp(wt, wt2, n * k) == 0);
    if (n % 4 == 0) oracle_pack_kmajor(p, n, k, pt);
    const float a = oracle_threshold_ternarize(w, n, k, 0.7f, wt2, &delta);
    CHECK(a >= 0.0f && delta >= 0.0f);
    oracle_quant_act(x, m, k, q, s);
    oracle_matmul_i32(q, m, k, wt, n, acc);
    oracle_rescale(acc, m, n, s, g, y);
    oracle_quant_act_a4(x, m, k, 1, q, s);
    oracle_quant_act_a4(x, m, k, k, q, s);
    oracle_quant_act_a4(x, m, k, (k + 1) / 2, q, s);
    oracle_matmul_i32(q, m, k, wt, n, acc);
    oracle_rescale_q(acc, m, n, s, g, 12.0f, y);
    for (int64_t i = 0; i < m * n; ++i) CHECK(isfinite(y[i]));
    free(w); free(x); free(wt); free(wt2); free(q); free(p); free(pt); free(acc); free(s); free(y);
}

int main(void)
{
    /* hand-worked case: gamma 0.625, bytes 0x92 0x25, acc [-112, 127] */
    const float w[8] = {0.5f, -1.0f, 0.125f, 2.0f, -0.3125f, 0.0f, 0.6875f, -0.375f};
    const float x[4] = {12.5f, -3.0f, 0.5f, -127.0f};
    int8_t wt[8], q[4];
    uint8_t p[2];
    int32_t acc[2];
    float s, y[2];
    CHECK(oracle_absmean(w, 2, 4) == 0.625f);
    oracle_ternarize(w, 2, 4, 0.625f, wt);
    oracle_pack(wt, 2, 4, p);
    CHECK(p[0] == 0x92 && p[1] == 0x25);
    oracle_quant_act(x, 1, 4, q, &s);
    oracle_matmul_i32(q, 1, 4, wt, 2, acc);
    CHECK(acc[0] == -112 && acc[1] == 127);
    oracle_rescale(acc, 1, 2, &s, 0.625f, y);
    CHECK(y[0] == -70.0f && y[1] == 79.375f);
    const uint8_t bad[2] = {0x55, 0xC0};
    CHECK(oracle_unpack(bad, 1, 8, wt) == 1);
    CHECK(oracle_e2m1_doubled(5.0f) == 8 && oracle_e2m1_doubled(-0.75f) == -2 && oracle_e2m1_doubled(100.0f) == 12);
    uint16_t hb[3] = {0x3F80, 0xC000, 0x0000};
    float hf[3];
    oracle_bf16_to_f32(hb, 3, hf);
    CHECK(hf[0] == 1.0f && hf[1] == -2.0f && hf[2] == 0.0f);
    float gg[3] = {2.0f, -1.0f, 0.0f}, uu[3] = {3.0f, 5.0f, 7.0f}, hh[3];
    oracle_sqrelu_gate(gg, uu, 3, hh);
    CHECK(hh[0] == 12.0f && hh[1] == 0.0f && hh[2] == 0.0f);
    /* degenerate and ragged shapes */
    run_linear(1, 4, 1, 0.02f, 0);
    run_linear(3, 260, 7, 0.02f, 1);
    run_linear(5, 64, 8, 0.0f, 0);      /* all-zero weights: gamma 0 */
    run_linear(17, 516, 36, 1.0f, 1);
    run_linear(2, 1028, 12, 1e-30f, 0); /* tiny weights */
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: ok\n");
    return 0;
}
