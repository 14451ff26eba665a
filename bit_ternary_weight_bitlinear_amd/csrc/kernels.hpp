// kernels.hpp -- host-side launchers of the gfx950 BitLinear kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// ---- weight packing (offline): gamma = mean|W| in fixed fp64 order, then codes
// workspace: n doubles (per-row sums)
hipError_t launch_pack(const float *w, int64_t n, int64_t k, uint8_t *packed, float *gamma,
                       double *rowsum, hipStream_t st);

// threshold quantizer: delta = factor * mean|W| (into delta[0]), codes sign(w) where
// |w| > delta, alpha = mean(|W| * mask); workspace: n doubles
hipError_t launch_pack_threshold(const float *w, int64_t n, int64_t k, float factor, uint8_t *packed,
                                 float *alpha, float *delta, double *rowsum, hipStream_t st);

// copies packed rows [n][k/4] into a zero-weight padded layout [n][kp/4] (code 1 in the tail)
hipError_t launch_pad_weights(const uint8_t *src, int64_t n, int64_t k, int64_t kp, uint8_t *dst,
                              hipStream_t st);

// ---- activation quantization, one workgroup per token.
// q_nat  (optional) int8 [m][k] natural layout
// q_perm (optional) int8 [m][kp] qperm layout, zero padded; then sumq[m] is written too
// s      fp32 [m]
hipError_t launch_act_quant(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp,
                            int8_t *q_nat, int8_t *q_perm, float *s, int32_t *sumq, hipStream_t st);

// the same after a per-token RMS normalization x^ = (x * r) * gain (gain optional, [k])
hipError_t launch_act_quant_norm(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp, const float *gain,
                                 int8_t *q_nat, int8_t *q_perm, float *s, int32_t *sumq, hipStream_t st);

// 4-bit activations: top-`keep` magnitudes per token kept, MinMax E2M1, codes stored
// doubled (2e in [-12, 12]) in the same outputs as launch_act_quant
hipError_t launch_act_quant_a4(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp, int64_t keep,
                               int8_t *q_nat, int8_t *q_perm, float *s, int32_t *sumq, hipStream_t st);

// int8 [m][k] natural -> qperm [m][kp] + sumq[m]
hipError_t launch_perm_q(const int8_t *q, int64_t m, int64_t k, int64_t kp, int8_t *q_perm,
                         int32_t *sumq, hipStream_t st);

// ---- decode GEMV (m <= 4) with the activation quantization fused in its prologue
struct GemvProblem {
    const void *x;
    bool bf16;
    int64_t m, k, kp, n;
    const uint8_t *w0, *w1;  // w1 != nullptr: gate/up pair, output h = relu(g)^2 * u
    int64_t ldw;             // bytes per packed row (kp / 4)
    const float *gamma0, *gamma1;
    float *out;              // y [m][n] or h [m][n]
    int32_t *acc_out;        // optional (single matrix only)
    int8_t *q_out;           // optional natural int8 copy of the quantized activations
    float *s_out;            // optional per-token scales
    const float *pre_s;      // quantized rows (the decode kernel): x holds qperm rows [m][kp]
    const int32_t *pre_sumq;
    float qmax = 127.0f;     // mode 2: code of the largest magnitude (127 int8, 12 doubled E2M1)
    float *hmax_part;        // gate/up pair, optional: max |h| per (workgroup, token), [grid][m]
    bool norm = false;       // RMS norm (subln) of the one bf16 token first (gemv_token_prologue_supported)
    const float *gain = nullptr;  // norm: per-input gain [k] or NULL
    bool a4 = false;         // 4-bit top-K E2M1 codes of the one bf16 token (gemv_token_prologue_supported); qmax = 12
    int64_t keep = 0;        // a4: entries kept
};
bool gemv_supported(int64_t m, int64_t kp);
// the decode kernel on quantized rows (pre_s set: x holds qperm rows [m][kp])
bool gemv_prequant_supported(int64_t m, int64_t kp);
// the decode kernel with the RMS norm or the 4-bit quantization in its
// prologue: one bf16 token, k % 16 == 0
bool gemv_token_prologue_supported(int64_t m, int64_t k, bool bf16);
// workgroups of a decode launch (the number of hmax_part rows it writes)
int64_t gemv_grid(int64_t n, int64_t kp, bool dual);
hipError_t launch_gemv(const GemvProblem &p, hipStream_t st);
// 5..16 tokens, single matrix, k <= 8192 (k % 16 == 0, m * k <= 32768):
// quantization, products and rescale in one launch (bgemv.hip)
bool bgemv_supported(int64_t m, int64_t k, bool bf16);
hipError_t launch_bgemv(const GemvProblem &p, hipStream_t st);

// ---- decode FFN down projection over the input-major weights, skipping the
// zero channels of the requantized h (sparse_down.hip)
// packed [n][k/4] -> input-major [k][n/4] (n % 4 == 0)
hipError_t launch_pack_kmajor(const uint8_t *packed, int64_t n, int64_t k, uint8_t *packed_t, hipStream_t st);
struct SparseDownProblem {
    const float *h;          // [m][ffn] fp32 (the gate/up launch's output)
    const float *hmax_part;  // [parts][m] partial maxima of |h|
    int64_t parts;
    int64_t m, ffn, hidden;
    const uint8_t *wt;       // input-major down weights [ffn][hidden/4]
    const float *gamma;
    float *y;                // [m][hidden]
    int32_t *partial;        // [sparse_down_partials()][m][hidden] int32 scratch
    float *s;                // [m] fp32 scratch (the row scales of h)
    int8_t *q_out;           // optional [m][ffn]
    float *s_out;            // optional [m]
};
int64_t sparse_down_nslices(int64_t hidden);
int64_t sparse_down_partials(int64_t hidden, int64_t ffn);
hipError_t launch_sparse_down(const SparseDownProblem &p, hipStream_t st);

// ---- MFMA GEMM on qperm activations
enum GemmEpilogue { EPI_Y = 0, EPI_ACC = 1, EPI_GATE = 2 };
struct GemmProblem {
    const int8_t *qp;  // [>= roundup(m, 256)][kp]
    int64_t kp;
    const float *s;
    const int32_t *sumq;
    int64_t m, n;
    const uint8_t *w0, *w1;
    int64_t ldw;
    const float *gamma0, *gamma1;
    float *out;        // EPI_Y: y; EPI_GATE: h
    int32_t *acc_out;  // EPI_Y: optional; EPI_ACC: required
    int epi;
    float qmax = 127.0f;  // code of the largest magnitude: 127 (int8) or 12 (doubled E2M1)
};
hipError_t launch_gemm(const GemmProblem &p, hipStream_t st);

// ---- 5..64 tokens: weight-streaming MFMA kernel, same problem description
bool skinny_supported(int64_t m);
hipError_t launch_skinny(const GemmProblem &p, hipStream_t st);

// ---- 1..64 tokens: row-tile x token-slice MFMA kernel with the token rows
// staged per wave in LDS (bmma.hip), same problem description; rows of up to
// 8192 inputs
bool bmma_supported(int64_t m, int64_t kp, bool dual);
hipError_t launch_bmma(const GemmProblem &p, hipStream_t st);

// MFMA path for m tokens: bmma up to 64 tokens (the skinny kernel for longer
// rows), the tiled GEMM above
inline hipError_t launch_contraction(const GemmProblem &p, hipStream_t st)
{
    if (bmma_supported(p.m, p.kp, p.epi == EPI_GATE)) return launch_bmma(p, st);
    return skinny_supported(p.m) ? launch_skinny(p, st) : launch_gemm(p, st);
}

}  // namespace bl
