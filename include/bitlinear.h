/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear library.
 *
 * The BitLinear layer replaces a bias-free nn.Linear ("穿越1比特的奇幻旅程",
 * summary of the BitNet b1.58 2B4T report, section 架构创新). The forward pass
 * computed here is the W1.58A8 product of that report's GPU inference section
 * (推理实现 / GPU端): ternary weights stored four per byte, int8 activations,
 * an int32 product, and a rescale back to fp32.
 *
 * Conventions shared by every call
 *  - Shapes follow nn.Linear: activations x are [m][k] (tokens x in-features),
 *    weights W are [n][k] (out-features x in-features), outputs y are [m][n].
 *    All arrays are dense and row-major.
 *  - Every pointer argument is a DEVICE pointer, except `stream`, which is a
 *    hipStream_t passed as void* (NULL = the null stream). Every call only
 *    enqueues work on `stream` and returns; nothing is synchronised, nothing is
 *    allocated, and the library keeps no mutable global state, so calls on
 *    different streams may run concurrently. The caller owns every buffer.
 *  - Outputs must not alias inputs. Device pointers must be 16-byte aligned.
 *  - Packed weight layout: row-major [n][k/4] bytes; byte j of a row holds the
 *    weights k = 4j+i in bits 2i..2i+1 (i = 0..3) as the code w+1 in {0,1,2};
 *    the code 3 never occurs.
 *  - Argument errors are reported before anything is enqueued. A failed kernel
 *    launch returns BL_ERR_HIP. Faults during execution surface at the
 *    caller's next synchronisation of `stream`. No C++ exception crosses the ABI.
 *  - The library targets gfx950 only.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BL_OK = 0,
    BL_ERR_NULL = 1,       /* a required pointer is NULL                        */
    BL_ERR_SHAPE = 2,      /* m, n < 1, k < 4, k % 4 != 0, or a size too large   */
    BL_ERR_ALIGN = 3,      /* a device pointer is not 16-byte aligned           */
    BL_ERR_DTYPE = 4,      /* unknown activation dtype                          */
    BL_ERR_WORKSPACE = 5,  /* workspace smaller than bitlinear_workspace_size() */
    BL_ERR_HIP = 6         /* a kernel launch failed                            */
} bl_status;

/* Element type of the activation input x. */
typedef enum { BL_F32 = 0, BL_BF16 = 1 } bl_dtype;

/* Operation selector for bitlinear_workspace_size(). */
typedef enum { BL_OP_PACK = 0, BL_OP_FORWARD = 1, BL_OP_FFN = 2, BL_OP_GEMM_I32 = 3 } bl_op;

/* Largest supported dimension (k, n, hidden, ffn) and token count m. */
#define BL_MAX_DIM ((int64_t)1 << 20)
#define BL_MAX_TOKENS ((int64_t)1 << 22)

/*
 * Bytes of device workspace an operation needs (0 if none), for
 *   BL_OP_PACK:      (m ignored, k, n)
 *   BL_OP_FORWARD:   (m, k, n)
 *   BL_OP_GEMM_I32:  (m, k, n)
 *   BL_OP_FFN:       (m, hidden, ffn)   -- the last two arguments
 * Returns 0 for invalid shapes as well; the operation itself then reports the
 * shape error.
 */
size_t bitlinear_workspace_size(int op, int64_t m, int64_t k, int64_t n);

/*
 * Offline weight quantization and packing ("BitNet 1-bit LLM 的混合精度微调技术",
 * BitLinear paragraph and operational-parameter paragraph: absmean scale;
 * "穿越1比特的奇幻旅程", sections 架构创新 and 推理实现 / GPU端: ternary values,
 * four per int8).
 *   w        fp32 [n][k] weights (input)
 *   packed   uint8 [n][k/4] 2-bit codes (output, layout above)
 *   gamma    fp32 [1] per-tensor scale gamma = mean|W| (output). The mean is
 *            accumulated in fp64: each row left to right, rows in order, then
 *            divided by n*k and rounded once to fp32. Weights quantize to
 *            clip(rint(w / gamma), -1, 1) with a correctly rounded fp32
 *            division and ties to even; gamma = 0 quantizes every weight to 0.
 *   workspace  >= bitlinear_workspace_size(BL_OP_PACK, 0, k, n) bytes.
 * Requires k % 4 == 0.
 */
bl_status bitlinear_pack_weights(const float *w, int64_t n, int64_t k,
                                 uint8_t *packed, float *gamma,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * Per-token absmax activation quantization to int8 ("BitNet 1-bit LLM 的混合精度
 * 微调技术", operational-parameter paragraph: absmax with epsilon 1e-5;
 * "BitNet 中使用直通估计器工程化三元权重训练", section 工程化训练流程与参数配置:
 * scale max|X| and factor 127; "穿越1比特的奇幻旅程", section 架构创新: 8-bit, per token).
 *   x        [m][k] activations of type `dtype` (BL_F32 or BL_BF16)
 *   q        int8 [m][k] (output): clamp(rint(x * (127 / s)), -127, 127)
 *   scale    fp32 [m] (output): s = max(max_k |x|, 1e-5)
 * Requires k % 4 == 0.
 */
bl_status bitlinear_quant_act(const void *x, int dtype, int64_t m, int64_t k,
                              int8_t *q, float *scale, void *stream);

/*
 * BitLinear forward: y = (x quantized per token) x (ternary W)^T, rescaled
 * ("穿越1比特的奇幻旅程", section 推理实现 / GPU端: the W1.58A8 matrix product).
 *   x        [m][k] activations of type `dtype`
 *   packed   uint8 [n][k/4], gamma fp32 [1]: output of bitlinear_pack_weights
 *   y        fp32 [m][n] (output): y = (float)acc * ((s / 127) * gamma)
 *   acc_out  optional int32 [m][n] (output): acc = sum_k q[m][k] * w~[n][k];
 *            NULL skips it
 *   workspace  >= bitlinear_workspace_size(BL_OP_FORWARD, m, k, n) bytes
 * Requires k % 4 == 0. No bias (the layer has none: section 架构创新).
 */
bl_status bitlinear_forward(const void *x, int dtype, int64_t m, int64_t k,
                            const uint8_t *packed, const float *gamma, int64_t n,
                            float *y, int32_t *acc_out,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Squared-ReLU gated FFN of three BitLinear layers ("穿越1比特的奇幻旅程", section
 * 架构创新: squared ReLU instead of SwiGLU; "BitNet 1-bit LLM 的混合精度微调技术",
 * operational-parameter paragraph: squared ReLU with GLU gating):
 *   q, s  = quant(x)                         (shared by gate and up)
 *   g, u  = BitLinear_gate(x), BitLinear_up(x)      fp32 [m][ffn]
 *   h     = (max(g,0) * max(g,0)) * u                fp32 [m][ffn]
 *   qh, sh = quant(h)                        (per-token int8 requantization)
 *   y     = BitLinear_down(h)                        fp32 [m][hidden]
 *   x            [m][hidden] of type `dtype`
 *   gate_packed, up_packed  uint8 [ffn][hidden/4];  down_packed uint8 [hidden][ffn/4]
 *   *_gamma      fp32 [1] each
 *   y            fp32 [m][hidden] (output)
 *   hq_out       optional int8 [m][ffn] (output): qh; NULL skips it
 *   hs_out       optional fp32 [m] (output): sh; NULL skips it
 *   workspace    >= bitlinear_workspace_size(BL_OP_FFN, m, hidden, ffn) bytes
 * Requires hidden % 4 == 0 and ffn % 4 == 0.
 */
bl_status bitlinear_ffn(const void *x, int dtype, int64_t m, int64_t hidden, int64_t ffn,
                        const uint8_t *gate_packed, const float *gate_gamma,
                        const uint8_t *up_packed, const float *up_gamma,
                        const uint8_t *down_packed, const float *down_gamma,
                        float *y, int8_t *hq_out, float *hs_out,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * The bare ternary x int8 contraction ("穿越1比特的奇幻旅程", section
 * 推理实现 / GPU端), exposed for parity checks of the integer product alone.
 *   q        int8 [m][k] (input, natural layout)
 *   packed   uint8 [n][k/4]
 *   acc      int32 [m][n] (output): sum_k q[m][k] * w~[n][k], exact
 *   workspace  >= bitlinear_workspace_size(BL_OP_GEMM_I32, m, k, n) bytes
 */
bl_status bitlinear_gemm_i32(const int8_t *q, int64_t m, int64_t k,
                             const uint8_t *packed, int64_t n, int32_t *acc,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *bitlinear_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
