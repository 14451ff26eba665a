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
 *    The one exception is bitlinear_forward_noalloc, which uses a
 *    library-owned scratch array per device (see there).
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
    BL_ERR_HIP = 6,        /* a kernel launch failed                            */
    BL_ERR_VALUE = 7,      /* a scalar argument is out of range                 */
    /* range sentinels, never returned: every int32 is a value of the type, so
       a caller may pass any int (the library reports unknown values) */
    BL_STATUS_RANGE_MIN_ = -0x7FFFFFFF - 1,
    BL_STATUS_RANGE_MAX_ = 0x7FFFFFFF
} bl_status;

/* Element type of the activation input x (other values: BL_ERR_DTYPE; the
   sentinels make every int32 a value of the type). */
typedef enum {
    BL_F32 = 0,
    BL_BF16 = 1,
    BL_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
    BL_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} bl_dtype;

/* Operation selector for bitlinear_workspace_size(): 0 = forward, 1 = FFN, as
 * the two calls a layer makes per batch; the offline pack and the bare integer
 * product follow. */
typedef enum {
    BL_OP_FORWARD = 0,
    BL_OP_FFN = 1,
    BL_OP_PACK = 2,
    BL_OP_GEMM_I32 = 3,
    BL_OP_PACK_THRESHOLD = 4,
    BL_OP_FORWARD_NORM = 5,
    BL_OP_FFN_SPARSE = 6,
    BL_OP_FORWARD_A4 = 7
} bl_op;

/* Largest supported dimension (k, n, hidden, ffn) and token count m. */
#define BL_MAX_DIM ((int64_t)1 << 20)
#define BL_MAX_TOKENS ((int64_t)1 << 22)

/*
 * Bytes of device workspace an operation needs (0 if none), for
 *   BL_OP_FORWARD:   (m, k, n)
 *   BL_OP_FFN:       (m, hidden, ffn)   -- the last two arguments
 *   BL_OP_PACK:      (m ignored, k, n)
 *   BL_OP_GEMM_I32:  (m, k, n)
 *   BL_OP_PACK_THRESHOLD: (m ignored, k, n)
 *   BL_OP_FORWARD_NORM:   (m, k, n)
 *   BL_OP_FFN_SPARSE:     (m, hidden, ffn)
 *   BL_OP_FORWARD_A4:     (m, k, n)
 * Returns 0 for invalid shapes and unknown ops as well; the operation itself
 * then reports the shape error.
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
 *   workspace  >= bitlinear_workspace_size(BL_OP_PACK, 0, k, n) bytes: the
 *            fp64 row sums of the fixed summation order (one per row), which
 *            the library may not allocate itself.
 * Requires k % 4 == 0.
 */
bl_status bitlinear_pack_weights(const float *w, int64_t n, int64_t k,
                                 uint8_t *packed, float *gamma,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * Offline weight quantization with a magnitude threshold ("BitNet 三元权重阈值
 * 优化工程实践", section on the core principle of ternary threshold optimization:
 * the threshold is a factor -- 0.7 by default, 0.6-0.75 per layer kind -- times
 * mean|W|; weights above it keep their sign, the rest become 0; the scale is
 * the mean of the kept magnitudes over the whole tensor).
 *   w             fp32 [n][k] weights (input)
 *   delta_factor  finite, >= 0 (else BL_ERR_VALUE)
 *   packed        uint8 [n][k/4] (output): the same 2-bit layout as
 *                 bitlinear_pack_weights, code = w~ + 1 with
 *                 w~ = sign(w) if |w| > delta (strict), else 0
 *   alpha         fp32 [1] (output): sum of |w| over the kept weights divided by
 *                 n*k (all weights), accumulated in fp64 in the fixed order of
 *                 bitlinear_pack_weights, rounded once to fp32. alpha takes
 *                 gamma's place in bitlinear_forward and bitlinear_ffn.
 *   delta_out     optional fp32 [1] (output): delta = delta_factor * mean|W| as
 *                 one fp32 product, mean|W| exactly as gamma above; NULL skips it
 *   workspace     >= bitlinear_workspace_size(BL_OP_PACK_THRESHOLD, 0, k, n) bytes
 * Requires k % 4 == 0.
 */
bl_status bitlinear_pack_weights_threshold(const float *w, int64_t n, int64_t k, float delta_factor,
                                           uint8_t *packed, float *alpha, float *delta_out,
                                           void *workspace, size_t workspace_bytes, void *stream);

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
bl_status bitlinear_quant_act(const void *x, bl_dtype dtype, int64_t m, int64_t k,
                              int8_t *q, float *scale, void *stream);

/*
 * Per-token RMS normalization fused into the absmax quantization: the
 * normalization BitLinear applies to its input before quantizing it ("subln",
 * "穿越1比特的奇幻旅程", section 架构创新: added for the stability of 1-bit
 * training; "BitNet 中使用直通估计器工程化三元权重训练", section
 * 工程化训练流程与参数配置: layer normalization keeping the variance, epsilon 1e-5).
 * The pages give no formula; the form used is RMSNorm without mean subtraction
 * or bias:
 *   S = sum_k x^2 (fp64, each square exact; the sum equals the correctly rounded
 *   fp64 sum except within ~k^2 2^-106 of a rounding boundary),
 *   r = 1 / sqrt(fp32(S / k) + 1e-5) in fp32, x^ = (x * r) * gain[k] in fp32,
 *   then q, scale as bitlinear_quant_act computes them for x^.
 *   gain     optional fp32 [k], 16-byte aligned; NULL = no gain (all ones)
 *   q, scale as in bitlinear_quant_act (scale = max(max_k |x^|, 1e-5))
 */
bl_status bitlinear_quant_act_norm(const void *x, bl_dtype dtype, int64_t m, int64_t k,
                                   const float *gain, int8_t *q, float *scale, void *stream);

/*
 * BitLinear forward of RMS-normalized activations: bitlinear_forward applied to
 * x^ of bitlinear_quant_act_norm, with the normalization fused into the
 * quantization kernel (no x^ in memory).
 *   gain       optional fp32 [k] (NULL = none)
 *   workspace  >= bitlinear_workspace_size(BL_OP_FORWARD_NORM, m, k, n) bytes
 * Other arguments and results as bitlinear_forward.
 */
bl_status bitlinear_forward_norm(const void *x, bl_dtype dtype, int64_t m, int64_t k, const float *gain,
                                 const uint8_t *packed, const float *gamma, int64_t n,
                                 float *y, int32_t *acc_out,
                                 void *workspace, size_t workspace_bytes, void *stream);

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
 * Cost note: the kernels read weight rows padded to a multiple of 64 inputs.
 * When k % 64 != 0 the workspace also holds such a padded copy of `packed`,
 * rewritten on every call (one extra n*k/4-byte read and write); the same
 * holds for bitlinear_ffn (hidden or ffn not a multiple of 64) and the
 * variants below.
 */
bl_status bitlinear_forward(const void *x, bl_dtype dtype, int64_t m, int64_t k,
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
bl_status bitlinear_ffn(const void *x, bl_dtype dtype, int64_t m, int64_t hidden, int64_t ffn,
                        const uint8_t *gate_packed, const float *gate_gamma,
                        const uint8_t *up_packed, const float *up_gamma,
                        const uint8_t *down_packed, const float *down_gamma,
                        float *y, int8_t *hq_out, float *hs_out,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * bitlinear_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc. Same
 * arguments and results as bitlinear_forward without the workspace: the
 * scratch space comes from a library-owned device array of
 * BL_NOALLOC_SCRATCH_BYTES per device, which each device the library runs on
 * holds until the process ends. Nothing is allocated, freed or synchronised.
 *   Returns BL_ERR_WORKSPACE when bitlinear_workspace_size(BL_OP_FORWARD, m, k, n)
 *   exceeds BL_NOALLOC_SCRATCH_BYTES (e.g. m * roundup(k, 64) above ~32 M);
 *   BL_ERR_VALUE when `stream` belongs to another device than the current one.
 * Every call on a device shares that device's array, and the array keeps the
 * last call's contents (every call writes what it reads first): calls that
 * overlap on one device race -- serialise them (one stream, or events).
 */
#define BL_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)
bl_status bitlinear_forward_noalloc(const void *x, bl_dtype dtype, int64_t m, int64_t k,
                                    const uint8_t *packed, const float *gamma, int64_t n,
                                    float *y, int32_t *acc_out, void *stream);

/*
 * 4-bit activations for the W1.58A4 variant ("BitNet 1-bit LLM 的混合精度微调技术",
 * paragraph on progressive quantization: activations brought to 4 bits in the
 * MinMax FP4 format with E2M1 bits, top-K sparsification of 50 % against
 * outlier channels). The pages give no formula; the form used, per token:
 *   tau  = the keep-th largest |x|; entries with |x| >= tau are kept (ties at
 *          tau all kept), the others become 0
 *   s    = max(max_k |x|, 1e-5); v = x * (6 / s) (one fp32 division per token)
 *   e    = the nearest E2M1 value to v (0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 *          negatives), ties to the value whose mantissa bit is 0
 *   q    = 2e, an int8 in [-12, 12], so that x ~ q * s / 12
 *   keep    1..k (BL_ERR_VALUE otherwise); the pages' 50 % is keep = ceil(k / 2)
 *   q, scale  int8 [m][k] and fp32 [m] (output)
 */
bl_status bitlinear_quant_act_a4(const void *x, bl_dtype dtype, int64_t m, int64_t k, int64_t keep,
                                 int8_t *q, float *scale, void *stream);

/*
 * W1.58A4 forward: the 4-bit codes of bitlinear_quant_act_a4 times the ternary
 * weights, y = (float)acc * ((s / 12) * gamma), acc = sum_k q[m][k] * w~[n][k]
 * (exact in int32: the doubled E2M1 codes are small integers).
 *   workspace  >= bitlinear_workspace_size(BL_OP_FORWARD_A4, m, k, n) bytes
 * Other arguments and results as bitlinear_forward.
 */
bl_status bitlinear_forward_a4(const void *x, bl_dtype dtype, int64_t m, int64_t k, int64_t keep,
                               const uint8_t *packed, const float *gamma, int64_t n,
                               float *y, int32_t *acc_out,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Input-major copy of packed weights (offline, once per weight): the codes of
 * packed [n][k/4] rearranged as packed_t [k][n/4], row c holding the codes of
 * outputs 4j+i of input c in bits 2i..2i+1 of byte j -- the packing of the
 * transposed ternary matrix. Used for the FFN's down projection by
 * bitlinear_ffn_sparse. Requires n % 4 == 0 and k % 4 == 0.
 */
bl_status bitlinear_pack_kmajor(const uint8_t *packed, int64_t n, int64_t k, uint8_t *packed_t, void *stream);

/*
 * bitlinear_ffn for decode (1 <= m <= 4 tokens) with the down projection reading
 * only the weights of the non-zero channels of the requantized h
 * ("BitNet 1-bit LLM 的混合精度微调技术", operational-parameter paragraph: with the
 * squared-ReLU GLU gating, only the non-zero channels are computed). The down
 * weights come input-major (bitlinear_pack_kmajor of the [hidden][ffn/4]
 * matrix), so a channel whose code is 0 for every token skips its whole row.
 * Results are those of bitlinear_ffn: zero codes contribute nothing.
 *   down_packed_t  uint8 [ffn][hidden/4] (input-major)
 *   workspace      >= bitlinear_workspace_size(BL_OP_FFN_SPARSE, m, hidden, ffn)
 * Other arguments as bitlinear_ffn. Requires m <= 4, hidden % 16 == 0 and
 * ffn % 4 == 0 (BL_ERR_SHAPE otherwise).
 */
bl_status bitlinear_ffn_sparse(const void *x, bl_dtype dtype, int64_t m, int64_t hidden, int64_t ffn,
                               const uint8_t *gate_packed, const float *gate_gamma,
                               const uint8_t *up_packed, const float *up_gamma,
                               const uint8_t *down_packed_t, const float *down_gamma,
                               float *y, int8_t *hq_out, float *hs_out,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * The bare ternary x int8 contraction ("穿越1比特的奇幻旅程", section
 * 推理实现 / GPU端), exposed for parity checks of the integer product alone.
 *   q        int8 [m][k] (input, natural layout)
 *   packed   uint8 [n][k/4]
 *   acc      int32 [m][n] (output): sum_k q[m][k] * w~[n][k], exact
 *   workspace  >= bitlinear_workspace_size(BL_OP_GEMM_I32, m, k, n) bytes: the
 *            kernels read q in an internal permuted layout, copied there first
 */
bl_status bitlinear_gemm_i32(const int8_t *q, int64_t m, int64_t k,
                             const uint8_t *packed, int64_t n, int32_t *acc,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *bitlinear_status_string(bl_status status);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
