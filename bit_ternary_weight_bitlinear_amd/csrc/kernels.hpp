// kernels.hpp -- host-side launchers of the gfx950 BitLinear kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// ---- weight packing (offline): gamma = mean|W| in fixed fp64 order, then codes
// workspace: n doubles (per-row sums)
hipError_t launch_pack(const float *w, int64_t n, int64_t k, uint8_t *packed, float *gamma,
                       double *rowsum, hipStream_t st);

// copies packed rows [n][k/4] into a zero-weight padded layout [n][kp/4] (code 1 in the tail)
hipError_t launch_pad_weights(const uint8_t *src, int64_t n, int64_t k, int64_t kp, uint8_t *dst,
                              hipStream_t st);

// ---- activation quantization, one workgroup per token.
// q_nat  (optional) int8 [m][k] natural layout
// q_perm (optional) int8 [m][kp] qperm layout, zero padded; then sumq[m] is written too
// s      fp32 [m]
hipError_t launch_act_quant(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp,
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
    const float *pre_s;      // 5..64-token kernel, mode 2 only (see bgemv_mode)
    const int32_t *pre_sumq;
};
bool gemv_supported(int64_t m, int64_t kp);
hipError_t launch_gemv(const GemvProblem &p, hipStream_t st);
// 5..64 tokens, single matrix, k <= 8192. Mode 1 (up to 16 tokens):
// quantization inside the launch; mode 2: x holds the qperm int8 rows
// [m][kp] of the quantization kernel and pre_s / pre_sumq its scales and
// sums; 0: neither (too many inputs for registers or LDS).
int bgemv_mode(int64_t m, int64_t k, bool bf16);
hipError_t launch_bgemv(const GemvProblem &p, hipStream_t st);

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
};
hipError_t launch_gemm(const GemmProblem &p, hipStream_t st);

// ---- 5..64 tokens: weight-streaming MFMA kernel, same problem description
bool skinny_supported(int64_t m);
hipError_t launch_skinny(const GemmProblem &p, hipStream_t st);

// MFMA path for m tokens: the skinny kernel up to 64 tokens, the tiled GEMM above
inline hipError_t launch_contraction(const GemmProblem &p, hipStream_t st)
{
    return skinny_supported(p.m) ? launch_skinny(p, st) : launch_gemm(p, st);
}

}  // namespace bl
