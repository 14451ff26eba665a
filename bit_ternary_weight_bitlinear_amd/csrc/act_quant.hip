// act_quant.hip -- per-token absmax int8 activation quantization for gfx950.
//
// s = max(max_k |x|, 1e-5), q = clamp(rint(x * (127 / s)), -127, 127)
// ("BitNet 1-bit LLM 的混合精度微调技术", operational-parameter paragraph: absmax with
// epsilon 1e-5; "BitNet 中使用直通估计器工程化三元权重训练", section
// 工程化训练流程与参数配置: scale max|X|, factor 127; "穿越1比特的奇幻旅程", section
// 架构创新: 8-bit, per token).
//
// One 256-thread workgroup per token. A thread owns 16-input groups; up to four
// groups per thread stay in registers between the absmax pass and the
// quantization pass (k <= 16384), longer rows are read twice. The number of
// resident groups is a template parameter sized to the row at launch, so short
// rows keep few registers and many tokens are in flight per CU. The absmax and
// the sum of the codes are reduced with DPP inside each wave and through LDS
// across the four waves. HBM-bound: it reads the row once and writes k bytes.
//
// NORM: an RMS normalization runs first (subln: "穿越1比特的奇幻旅程", section
// 架构创新; layer normalization with epsilon 1e-5: "BitNet 中使用直通估计器工程化
// 三元权重训练", section 工程化训练流程与参数配置), and the absmax quantization
// then applies to x^ = (x * r) * g, r = 1 / sqrt(fp32(S / k) + 1e-5), with
// S = sum of x^2. Every square is exact in fp64; the sum is kept as a
// double-double (TwoSum: each addition's rounding error is carried exactly),
// so hi + lo rounds to the correctly rounded S unless S lies within about
// k^2 2^-106 of a rounding boundary of fp64. The fp32 steps after it are
// single correctly rounded operations (no contraction in this build).
//
// A4 (act_quant_a4_kernel): 4-bit activations ("BitNet 1-bit LLM 的混合精度微调
// 技术", paragraph on progressive quantization: MinMax FP4 with E2M1 bits, top-K
// sparsification of 50 %). Per token, the keep-th largest magnitude tau is
// found by a radix select on the fp32 bits of |x| (non-negative floats order
// like their bit patterns) with 11-bit digits from the top: each pass builds a
// 2048-bin histogram of the candidates' digit in LDS, and every wave scans it
// on its own for the digit that holds the keep-th largest (two passes for
// bf16, whose low 16 bits are zero; three for fp32). Entries with |x| >= tau
// are kept, v = x * (6 / s) with s = max(max|x|, 1e-5), and v goes to the
// nearest E2M1 value (ties to the even mantissa), stored doubled as an int8
// code in [-12, 12].
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

__device__ inline float block_max(float v, float *red)
{
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ inline int block_sum(int v, int *red)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// natural-order store of group g: inputs 16g .. min(16g+16, k) (k % 4 == 0, rows 4-byte aligned)
__device__ inline void store_nat(int8_t *row, int64_t k, int64_t g, const uint4 v)
{
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t *p = reinterpret_cast<uint32_t *>(row + 16 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (16 * g + 4 * j < k) p[j] = d[j];
}

// x^ = (x * r) * g for the 16 inputs of group g (gain entries past k unused)
template <bool GAIN>
__device__ inline void normalize_group(float f[16], float r, const float *gain, int64_t k, int64_t g)
{
    const int64_t k0 = 16 * g;
#pragma unroll
    for (int j = 0; j < 16; ++j) f[j] = f[j] * r;
    if constexpr (GAIN) {
        if (k0 + 16 <= k) {
            const float4 *gp = reinterpret_cast<const float4 *>(gain + k0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 gv = gp[j];
                f[4 * j + 0] = f[4 * j + 0] * gv.x;
                f[4 * j + 1] = f[4 * j + 1] * gv.y;
                f[4 * j + 2] = f[4 * j + 2] * gv.z;
                f[4 * j + 3] = f[4 * j + 3] * gv.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) f[j] = (k0 + j < k) ? f[j] * gain[k0 + j] : 0.0f;
        }
    }
}

}  // namespace

constexpr int kResidentGroups = 4;

// NORM = 0: plain absmax quantization; 1: RMS norm first, no gain; 2: RMS norm
// with the per-channel gain `gain` [k]
template <typename T, bool FULL, int RG, int NORM = 0>
__global__ __launch_bounds__(256) void act_quant_kernel(const T *__restrict__ x, int64_t k, int64_t kp,
                                                        int8_t *__restrict__ q_nat,
                                                        int8_t *__restrict__ q_perm,
                                                        float *__restrict__ s, int32_t *__restrict__ sumq,
                                                        const float *__restrict__ gain)
{
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    __shared__ double red_d[8];
    const int64_t t = blockIdx.x;
    const T *row = x + t * k;
    const int64_t G = ceil_div(k, 16);
    const bool resident = G <= (int64_t)RG * kThreads;

    // a group as the quantizer sees it: the inputs, normalized when NORM is set
    float r_norm = 1.0f;
    auto load = [&](int64_t g, float f[16]) {
        load_group<T, FULL>(row, k, g, f);
        if constexpr (NORM != 0) normalize_group<NORM == 2>(f, r_norm, gain, k, g);
    };

    float v[RG][16];
    if constexpr (NORM != 0) {
        double hi = 0.0, lo = 0.0;
        auto sq = [&](const float f[16]) {
#pragma unroll
            for (int j = 0; j < 16; ++j) dd_add(hi, lo, (double)f[j] * (double)f[j]);
        };
        if (resident) {
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const int64_t g = threadIdx.x + r * kThreads;
                if (g < G) {
                    load_group<T, FULL>(row, k, g, v[r]);
                    sq(v[r]);
                }
            }
        } else {
            for (int64_t g = threadIdx.x; g < G; g += kThreads) {
                float f[16];
                load_group<T, FULL>(row, k, g, f);
                sq(f);
            }
        }
        r_norm = norm_factor(block_sum_dd<4>(hi, lo, red_d), k);
    }
    float amax = 0.0f;
    if (resident) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int64_t g = threadIdx.x + r * kThreads;
            if (g < G) {
                if constexpr (NORM == 0) load_group<T, FULL>(row, k, g, v[r]);
                else normalize_group<NORM == 2>(v[r], r_norm, gain, k, g);
#pragma unroll
                for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[r][j]));
            }
        }
    } else {
        for (int64_t g = threadIdx.x; g < G; g += kThreads) {
            float f[16];
            load(g, f);
#pragma unroll
            for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(f[j]));
        }
    }
    amax = block_max(amax, red_f);
    const float st = fmaxf(amax, kEps);
    const float inv = 127.0f / st;

    int qsum = 0;
    auto emit = [&](int64_t g, const float f[16]) {
        uint4 pv, nv;
        qsum += quant_group(f, inv, &pv, &nv);
        if (q_perm) *reinterpret_cast<uint4 *>(q_perm + t * kp + 16 * g) = pv;
        if (q_nat) store_nat(q_nat + t * k, k, g, nv);
    };
    if (resident) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int64_t g = threadIdx.x + r * kThreads;
            if (g < G) emit(g, v[r]);
        }
    } else {
        for (int64_t g = threadIdx.x; g < G; g += kThreads) {
            float f[16];
            load(g, f);
            emit(g, f);
        }
    }
    if (q_perm) {
        for (int64_t g = G + threadIdx.x; g < kp / 16; g += kThreads)
            *reinterpret_cast<uint4 *>(q_perm + t * kp + 16 * g) = make_uint4(0, 0, 0, 0);
        const int total = block_sum(qsum, red_i);
        if (threadIdx.x == 0) sumq[t] = total;
    }
    if (threadIdx.x == 0) s[t] = st;
}

// 4-bit activations: one workgroup per token, 256 threads, as act_quant_kernel
template <typename T, bool FULL, int RG>
__global__ __launch_bounds__(256) void act_quant_a4_kernel(const T *__restrict__ x, int64_t k, int64_t kp,
                                                           int64_t keep, int8_t *__restrict__ q_nat,
                                                           int8_t *__restrict__ q_perm, float *__restrict__ s,
                                                           int32_t *__restrict__ sumq)
{
    constexpr int LOW = sizeof(T) == 2 ? 16 : 0;  // bf16: the low 16 bits are zero
    constexpr int PASSES = (31 - LOW + kDigitBits - 1) / kDigitBits;
    __shared__ __align__(16) int hist[PASSES][kDigitBins];
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    const int64_t t = blockIdx.x;
    const T *row = x + t * k;
    const int64_t G = ceil_div(k, 16);
    const bool resident = G <= (int64_t)RG * kThreads;

    for (int i = threadIdx.x; i < PASSES * kDigitBins / 4; i += kThreads)
        reinterpret_cast<int4 *>(&hist[0][0])[i] = make_int4(0, 0, 0, 0);

    float v[RG][16];
    float amax = 0.0f;
    if (resident) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int64_t g = threadIdx.x + r * kThreads;
            if (g < G) {
                load_group<T, FULL>(row, k, g, v[r]);
#pragma unroll
                for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[r][j]));
            }
        }
    } else {
        for (int64_t g = threadIdx.x; g < G; g += kThreads) {
            float f[16];
            load_group<T, FULL>(row, k, g, f);
#pragma unroll
            for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(f[j]));
        }
    }
    amax = block_max(amax, red_f);

    // radix select of tau, the keep-th largest |x|: bits 30..20, then 19..16
    // for bf16 (19..9 and 8..0 for fp32). Inputs past k (the zero padding of
    // the last group) are not candidates. The barrier in block_max above also
    // publishes the zeroed histograms.
    uint32_t prefix = 0, pmask = 0;
    int want = (int)keep;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int hi = 31 - p * kDigitBits;
        const int lo = hi - kDigitBits > LOW ? hi - kDigitBits : LOW;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        int *h = hist[p];
        auto count = [&](const float f[16], int64_t g) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t key = __float_as_uint(fabsf(f[j]));
                if ((FULL || 16 * g + j < k) && (key & pmask) == prefix) atomicAdd(&h[(key >> lo) & dmask], 1);
            }
        };
        if (resident) {
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const int64_t g = threadIdx.x + r * kThreads;
                if (g < G) count(v[r], g);
            }
        } else {
            for (int64_t g = threadIdx.x; g < G; g += kThreads) {
                float f[16];
                load_group<T, FULL>(row, k, g, f);
                count(f, g);
            }
        }
        __syncthreads();
        prefix |= pick_digit(h, want) << lo;
        pmask |= dmask << lo;
    }
    const uint32_t tau = prefix;  // the keep-th largest |x| (as bits)
    const float st = fmaxf(amax, kEps);
    const float inv = 6.0f / st;

    int qsum = 0;
    auto emit = [&](int64_t g, const float f[16]) {
        int qi[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            qi[j] = __float_as_uint(fabsf(f[j])) >= tau ? e2m1_doubled(f[j] * inv) : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) qsum += qi[j];
        if (q_perm) *reinterpret_cast<uint4 *>(q_perm + t * kp + 16 * g) = qperm_pack(qi);
        if (q_nat) {
            uint32_t d[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                d[i] = (uint32_t)(qi[4 * i] & 0xFF) | ((uint32_t)(qi[4 * i + 1] & 0xFF) << 8) |
                       ((uint32_t)(qi[4 * i + 2] & 0xFF) << 16) | ((uint32_t)(qi[4 * i + 3] & 0xFF) << 24);
            store_nat(q_nat + t * k, k, g, make_uint4(d[0], d[1], d[2], d[3]));
        }
    };
    if (resident) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int64_t g = threadIdx.x + r * kThreads;
            if (g < G) emit(g, v[r]);
        }
    } else {
        for (int64_t g = threadIdx.x; g < G; g += kThreads) {
            float f[16];
            load_group<T, FULL>(row, k, g, f);
            emit(g, f);
        }
    }
    if (q_perm) {
        for (int64_t g = G + threadIdx.x; g < kp / 16; g += kThreads)
            *reinterpret_cast<uint4 *>(q_perm + t * kp + 16 * g) = make_uint4(0, 0, 0, 0);
        const int total = block_sum(qsum, red_i);
        if (threadIdx.x == 0) sumq[t] = total;
    }
    if (threadIdx.x == 0) s[t] = st;
}

template <typename T, bool FULL, int NORM>
static void launch_rg(const T *x, int64_t m, int64_t k, int64_t kp, int8_t *q_nat, int8_t *q_perm, float *s,
                      int32_t *sumq, const float *gain, hipStream_t st)
{
    const dim3 grid((unsigned)m), block(kThreads);
    const int64_t groups = ceil_div(k, 16);
    const int64_t rg = ceil_div(groups, kThreads);
    if (rg <= 1)
        hipLaunchKernelGGL((act_quant_kernel<T, FULL, 1, NORM>), grid, block, 0, st, x, k, kp, q_nat, q_perm, s,
                           sumq, gain);
    else if (rg == 2)
        hipLaunchKernelGGL((act_quant_kernel<T, FULL, 2, NORM>), grid, block, 0, st, x, k, kp, q_nat, q_perm, s,
                           sumq, gain);
    else
        hipLaunchKernelGGL((act_quant_kernel<T, FULL, kResidentGroups, NORM>), grid, block, 0, st, x, k, kp, q_nat,
                           q_perm, s, sumq, gain);
}

template <int NORM>
static void launch_any(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp, int8_t *q_nat,
                       int8_t *q_perm, float *s, int32_t *sumq, const float *gain, hipStream_t st)
{
    const bool full = k % 16 == 0;
    if (bf16) {
        const bf16_t *xb = static_cast<const bf16_t *>(x);
        if (full) launch_rg<bf16_t, true, NORM>(xb, m, k, kp, q_nat, q_perm, s, sumq, gain, st);
        else launch_rg<bf16_t, false, NORM>(xb, m, k, kp, q_nat, q_perm, s, sumq, gain, st);
    } else {
        const float *xf = static_cast<const float *>(x);
        if (full) launch_rg<float, true, NORM>(xf, m, k, kp, q_nat, q_perm, s, sumq, gain, st);
        else launch_rg<float, false, NORM>(xf, m, k, kp, q_nat, q_perm, s, sumq, gain, st);
    }
}

hipError_t launch_act_quant(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp, int8_t *q_nat,
                            int8_t *q_perm, float *s, int32_t *sumq, hipStream_t st)
{
    launch_any<0>(x, bf16, m, k, kp, q_nat, q_perm, s, sumq, nullptr, st);
    return hipGetLastError();
}

template <typename T, bool FULL>
static void launch_a4_rg(const T *x, int64_t m, int64_t k, int64_t kp, int64_t keep, int8_t *q_nat, int8_t *q_perm,
                         float *s, int32_t *sumq, hipStream_t st)
{
    const dim3 grid((unsigned)m), block(kThreads);
    const int64_t rg = ceil_div(ceil_div(k, 16), kThreads);
    if (rg <= 1)
        hipLaunchKernelGGL((act_quant_a4_kernel<T, FULL, 1>), grid, block, 0, st, x, k, kp, keep, q_nat, q_perm, s,
                           sumq);
    else if (rg == 2)
        hipLaunchKernelGGL((act_quant_a4_kernel<T, FULL, 2>), grid, block, 0, st, x, k, kp, keep, q_nat, q_perm, s,
                           sumq);
    else
        hipLaunchKernelGGL((act_quant_a4_kernel<T, FULL, kResidentGroups>), grid, block, 0, st, x, k, kp, keep,
                           q_nat, q_perm, s, sumq);
}

hipError_t launch_act_quant_a4(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp, int64_t keep,
                               int8_t *q_nat, int8_t *q_perm, float *s, int32_t *sumq, hipStream_t st)
{
    const bool full = k % 16 == 0;
    if (bf16) {
        const bf16_t *xb = static_cast<const bf16_t *>(x);
        if (full) launch_a4_rg<bf16_t, true>(xb, m, k, kp, keep, q_nat, q_perm, s, sumq, st);
        else launch_a4_rg<bf16_t, false>(xb, m, k, kp, keep, q_nat, q_perm, s, sumq, st);
    } else {
        const float *xf = static_cast<const float *>(x);
        if (full) launch_a4_rg<float, true>(xf, m, k, kp, keep, q_nat, q_perm, s, sumq, st);
        else launch_a4_rg<float, false>(xf, m, k, kp, keep, q_nat, q_perm, s, sumq, st);
    }
    return hipGetLastError();
}

hipError_t launch_act_quant_norm(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp, const float *gain,
                                 int8_t *q_nat, int8_t *q_perm, float *s, int32_t *sumq, hipStream_t st)
{
    if (gain) launch_any<2>(x, bf16, m, k, kp, q_nat, q_perm, s, sumq, gain, st);
    else launch_any<1>(x, bf16, m, k, kp, q_nat, q_perm, s, sumq, nullptr, st);
    return hipGetLastError();
}

// natural int8 [m][k] -> qperm [m][kp] and sumq (for the bare integer product)
__global__ __launch_bounds__(256) void perm_q_kernel(const int8_t *__restrict__ q, int64_t k, int64_t kp,
                                                     int8_t *__restrict__ q_perm,
                                                     int32_t *__restrict__ sumq)
{
    __shared__ int red_i[4];
    const int64_t t = blockIdx.x;
    const int8_t *row = q + t * k;
    int qsum = 0;
    for (int64_t g = threadIdx.x; g < kp / 16; g += kThreads) {
        int qi[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t k0 = 16 * g + 4 * j;
            const uint32_t d = k0 < k ? *reinterpret_cast<const uint32_t *>(row + k0) : 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) qi[4 * j + b] = (int)(int8_t)(d >> (8 * b));
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) qsum += qi[j];
        *reinterpret_cast<uint4 *>(q_perm + t * kp + 16 * g) = qperm_pack(qi);
    }
    const int total = block_sum(qsum, red_i);
    if (threadIdx.x == 0) sumq[t] = total;
}

hipError_t launch_perm_q(const int8_t *q, int64_t m, int64_t k, int64_t kp, int8_t *q_perm,
                         int32_t *sumq, hipStream_t st)
{
    hipLaunchKernelGGL(perm_q_kernel, dim3((unsigned)m), dim3(kThreads), 0, st, q, k, kp, q_perm, sumq);
    return hipGetLastError();
}

}  // namespace bl
