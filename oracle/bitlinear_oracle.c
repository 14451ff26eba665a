/*
 * bitlinear_oracle.c -- plain CPU oracle for the BitNet b1.58 BitLinear forward
 * pass (W1.58A8). TEST INFRASTRUCTURE ONLY: this file is used by the tests, the
 * smoke check and the benchmark's CPU-baseline leg. The product path never
 * links, loads or calls it, and it shares no code with the HIP library.
 *
 * Sources (cited by page title and section):
 *  [P1] "BitNet 1-bit LLM 的混合精度微调技术：渐进量化策略" (blog.hotdry.top,
 *       2025-10-07), body paragraph on the BitLinear layer and the paragraph
 *       on operational parameters (quantization functions).
 *  [P2] "BitNet 中使用直通估计器工程化三元权重训练" (blog.hotdry.top, 2025-10-04),
 *       section "工程化训练流程与参数配置", activation-quantization item.
 *  [P3] "穿越1比特的奇幻旅程：高效语言模型的未来之谜" (beiduofen.top; summary of
 *       the BitNet b1.58 2B4T Technical Report), sections "架构创新" and
 *       "推理实现 / GPU端".
 *  [P4] "BitNet 三元权重阈值优化工程实践" (blog.hotdry.top, 2025-09-08), section
 *       on the core principle of ternary threshold optimization (the threshold
 *       quantizer and its code).
 *  [P1'] [P1], the paragraph on progressive quantization (second stage: 4-bit
 *       activations in the MinMax FP4 format with E2M1 bits, top-K
 *       sparsification of 50 % for outlier channels).
 *
 * Every function is a direct loop over the definition. Floating point follows
 * the precision the kernels decide integers in (fp32), with the operation order
 * fixed below; the weight-scale reduction accumulates in fp64.
 *
 * Readings where the pages leave the step open:
 *  - weight quantizer: absmean RoundClip with one per-tensor scale gamma [P1, P3];
 *  - ties round half to even (rintf under the default rounding mode);
 *  - gamma = 0 (all-zero weight) stores gamma = 0 and every weight quantizes to 0;
 *  - gamma is summed in fp64, row by row (each row left to right), rows in order;
 *  - codes come from a correctly rounded fp32 division w / gamma;
 *  - activation scale s = max(max|x|, 1e-5) and q = rint(x * (127 / s)),
 *    clamped to [-127, 127]; the stored per-token scale is s;
 *  - output y = (float)acc * ((s / 127) * gamma), in that order;
 *  - 2-bit code = w + 1, four codes per byte, k = 4j + i in bits 2i..2i+1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_EPS 1e-5f

/* Number of threads the contraction loops use (for the benchmark's report). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int t)
{
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}

/* bf16 -> fp32 widening: the bf16 bits are the upper half of the fp32 bits. */
void oracle_bf16_to_f32(const uint16_t *x, int64_t count, float *out)
{
    for (int64_t i = 0; i < count; ++i) {
        uint32_t bits = ((uint32_t)x[i]) << 16;
        memcpy(&out[i], &bits, sizeof bits);
    }
}

/* gamma = mean |W| over the whole tensor (absmean scale) [P1 operational
 * parameters; P3 架构创新]. fp64 accumulation: each row is summed left to right,
 * the row sums are added in row order, the total is divided by n*k and rounded
 * once to fp32. */
float oracle_absmean(const float *w, int64_t n, int64_t k)
{
    double total = 0.0;
    for (int64_t r = 0; r < n; ++r) {
        double row = 0.0;
        for (int64_t c = 0; c < k; ++c)
            row += fabs((double)w[r * k + c]);
        total += row;
    }
    return (float)(total / ((double)n * (double)k));
}

/* RoundClip(W / gamma, -1, 1): divide by the absmean scale, round to the nearest
 * integer, clip to [-1, 1] [P1 BitLinear paragraph]. */
void oracle_ternarize(const float *w, int64_t n, int64_t k, float gamma, int8_t *wt)
{
    for (int64_t i = 0; i < n * k; ++i) {
        float t = (gamma > 0.0f) ? w[i] / gamma : 0.0f;
        float r = rintf(t);
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        wt[i] = (int8_t)r;
    }
}

/* Threshold ternarization [P4, section on the core principle]: a weight is kept
 * (as its sign) when its magnitude exceeds delta = factor * mean|W|, and the
 * layer's scale is the mean over all n*k weights of |w| times that mask.
 * Readings: mean|W| is the absmean above (same fixed fp64 order, one fp32
 * rounding); delta is the fp32 product factor * mean; the mask is a strict
 * |w| > delta in fp32; the masked magnitudes are summed in fp64 in the same
 * fixed order as the absmean and divided by n*k (not by the number kept),
 * then rounded once to fp32. Writes the ternary weights and delta; returns
 * the scale alpha. */
float oracle_threshold_ternarize(const float *w, int64_t n, int64_t k, float factor, int8_t *wt,
                                 float *delta_out)
{
    const float mean = oracle_absmean(w, n, k);
    const float delta = factor * mean;
    double total = 0.0;
    for (int64_t r = 0; r < n; ++r) {
        double row = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            const float v = w[r * k + c];
            const float a = fabsf(v);
            if (a > delta) {
                row += (double)a;
                wt[r * k + c] = (int8_t)((v > 0.0f) - (v < 0.0f));
            } else {
                wt[r * k + c] = 0;
            }
        }
        total += row;
    }
    *delta_out = delta;
    const double kept_mean = total / ((double)n * (double)k);
    return (float)kept_mean;
}

/* Four ternary weights per byte [P3 推理实现 / GPU端]; code = w + 1 in {0,1,2};
 * row-major [n][k/4]; weight k = 4j + i of a row sits in bits 2i..2i+1 of byte j. */
void oracle_pack(const int8_t *wt, int64_t n, int64_t k, uint8_t *packed)
{
    const int64_t kb = k / 4;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < kb; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                unsigned code = (unsigned)(wt[r * k + 4 * j + i] + 1);
                byte |= code << (2 * i);
            }
            packed[r * kb + j] = (uint8_t)byte;
        }
}

/* The same weights in the input-major ("K-major") order: the packing of the
 * transposed ternary matrix. Row c of the output (one input feature) holds the
 * codes of outputs r = 4j + i in bits 2i..2i+1 of byte j. Needs n % 4 == 0. */
void oracle_pack_kmajor(const uint8_t *packed, int64_t n, int64_t k, uint8_t *out)
{
    const int64_t kb = k / 4, nb = n / 4;
    for (int64_t c = 0; c < k; ++c)
        for (int64_t j = 0; j < nb; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                const int64_t r = 4 * j + i;
                const unsigned code_r = (packed[r * kb + c / 4] >> (2 * (c % 4))) & 3u;
                byte |= code_r << (2 * i);
            }
            out[c * nb + j] = (uint8_t)byte;
        }
}

/* Inverse of oracle_pack. Returns the number of invalid codes (3) found; those
 * positions are written as 0. */
int64_t oracle_unpack(const uint8_t *packed, int64_t n, int64_t k, int8_t *wt)
{
    const int64_t kb = k / 4;
    int64_t bad = 0;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < kb; ++j)
            for (int i = 0; i < 4; ++i) {
                unsigned code = (packed[r * kb + j] >> (2 * i)) & 3u;
                if (code == 3u) { ++bad; wt[r * k + 4 * j + i] = 0; }
                else wt[r * k + 4 * j + i] = (int8_t)((int)code - 1);
            }
    return bad;
}

/* Per-token absmax quantization to int8 [P1 BitLinear and operational-parameter
 * paragraphs (epsilon 1e-5); P2 activation item (scale = max|X|, factor 127);
 * P3 架构创新 (8-bit, per token, absmax)]. */
void oracle_quant_act(const float *x, int64_t m, int64_t k, int8_t *q, float *s)
{
    for (int64_t t = 0; t < m; ++t) {
        const float *row = x + t * k;
        float amax = 0.0f;
        for (int64_t c = 0; c < k; ++c) {
            float a = fabsf(row[c]);
            if (a > amax) amax = a;
        }
        float st = amax > ORACLE_EPS ? amax : ORACLE_EPS;
        float inv = 127.0f / st;
        for (int64_t c = 0; c < k; ++c) {
            float v = rintf(row[c] * inv);
            if (v > 127.0f) v = 127.0f;
            if (v < -127.0f) v = -127.0f;
            q[t * k + c] = (int8_t)v;
        }
        s[t] = st;
    }
}

/* Nearest E2M1 value of v (the FP4 grid 0, 0.5, 1, 1.5, 2, 3, 4, 6 and its
 * negatives), returned doubled as an integer in [-12, 12]. Ties go to the value
 * whose mantissa bit is 0 (0, 1, 2, 4): round half to even on that grid. */
int oracle_e2m1_doubled(float v)
{
    const float a = fabsf(v);
    int c;
    if (a <= 0.25f) c = 0;
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;
    else if (a < 3.5f) c = 6;
    else if (a <= 5.0f) c = 8;
    else c = 12;
    return v < 0.0f ? -c : c;
}

static int desc_float(const void *pa, const void *pb)
{
    const float a = *(const float *)pa, b = *(const float *)pb;
    return (a < b) - (a > b);
}

/* 4-bit activations [P1']: per token, the entries whose magnitude is at least
 * the keep-th largest magnitude are kept (top-K; entries tied with that value
 * are all kept), the rest become 0; the kept entries are scaled so that the
 * largest magnitude s = max(max|x|, 1e-5) maps to 6, the largest E2M1 value
 * (MinMax), v = x * (6 / s) with one fp32 division per token, and rounded to
 * the nearest E2M1 value. q holds the doubled value 2e (an integer in
 * [-12, 12], so q * s / 12 approximates x); s is stored per token. */
void oracle_quant_act_a4(const float *x, int64_t m, int64_t k, int64_t keep, int8_t *q, float *s)
{
    float *mag = (float *)malloc((size_t)k * sizeof(float));
    for (int64_t t = 0; t < m; ++t) {
        const float *row = x + t * k;
        for (int64_t c = 0; c < k; ++c) mag[c] = fabsf(row[c]);
        qsort(mag, (size_t)k, sizeof(float), desc_float);
        const float tau = mag[keep - 1];
        const float amax = mag[0];
        const float st = amax > ORACLE_EPS ? amax : ORACLE_EPS;
        const float inv = 6.0f / st;
        for (int64_t c = 0; c < k; ++c)
            q[t * k + c] = fabsf(row[c]) >= tau ? (int8_t)oracle_e2m1_doubled(row[c] * inv) : 0;
        s[t] = st;
    }
    free(mag);
}

/* acc[t][r] = sum_c q[t][c] * wt[r][c], exact in int32 (the W1.58A8 product,
 * [P3 推理实现 / GPU端]). */
void oracle_matmul_i32(const int8_t *q, int64_t m, int64_t k,
                       const int8_t *wt, int64_t n, int32_t *acc)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < m; ++t)
        for (int64_t r = 0; r < n; ++r) {
            int32_t sum = 0;
            for (int64_t c = 0; c < k; ++c)
                sum += (int32_t)q[t * k + c] * (int32_t)wt[r * k + c];
            acc[t * n + r] = sum;
        }
}

/* y = acc * gamma * s / qmax: undo both quantization scales (qmax = 127 for
 * the int8 codes, 12 for the doubled E2M1 codes). */
void oracle_rescale_q(const int32_t *acc, int64_t m, int64_t n,
                      const float *s, float gamma, float qmax, float *y)
{
    for (int64_t t = 0; t < m; ++t) {
        const float ct = (s[t] / qmax) * gamma;
        for (int64_t r = 0; r < n; ++r)
            y[t * n + r] = (float)acc[t * n + r] * ct;
    }
}

/* y = acc * gamma * s / 127: undo both quantization scales. */
void oracle_rescale(const int32_t *acc, int64_t m, int64_t n,
                    const float *s, float gamma, float *y)
{
    for (int64_t t = 0; t < m; ++t) {
        float c = (s[t] / 127.0f) * gamma;
        for (int64_t r = 0; r < n; ++r)
            y[t * n + r] = (float)acc[t * n + r] * c;
    }
}

/* Squared-ReLU gating of the FFN: h = relu(g)^2 * u [P3 架构创新; P1 operational
 * parameters (squared ReLU with GLU gating)]. */
void oracle_sqrelu_gate(const float *g, const float *u, int64_t count, float *h)
{
    for (int64_t i = 0; i < count; ++i) {
        float gp = g[i] > 0.0f ? g[i] : 0.0f;
        h[i] = (gp * gp) * u[i];
    }
}
