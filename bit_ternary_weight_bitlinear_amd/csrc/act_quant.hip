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

}  // namespace

constexpr int kResidentGroups = 4;

template <typename T, bool FULL, int RG>
__global__ __launch_bounds__(256) void act_quant_kernel(const T *__restrict__ x, int64_t k, int64_t kp,
                                                        int8_t *__restrict__ q_nat,
                                                        int8_t *__restrict__ q_perm,
                                                        float *__restrict__ s, int32_t *__restrict__ sumq)
{
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    const int64_t t = blockIdx.x;
    const T *row = x + t * k;
    const int64_t G = ceil_div(k, 16);
    const bool resident = G <= (int64_t)RG * kThreads;

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

template <typename T, bool FULL>
static void launch_rg(const T *x, int64_t m, int64_t k, int64_t kp, int8_t *q_nat, int8_t *q_perm, float *s,
                      int32_t *sumq, hipStream_t st)
{
    const dim3 grid((unsigned)m), block(kThreads);
    const int64_t groups = ceil_div(k, 16);
    const int64_t rg = ceil_div(groups, kThreads);
    if (rg <= 1)
        hipLaunchKernelGGL((act_quant_kernel<T, FULL, 1>), grid, block, 0, st, x, k, kp, q_nat, q_perm, s, sumq);
    else if (rg == 2)
        hipLaunchKernelGGL((act_quant_kernel<T, FULL, 2>), grid, block, 0, st, x, k, kp, q_nat, q_perm, s, sumq);
    else
        hipLaunchKernelGGL((act_quant_kernel<T, FULL, kResidentGroups>), grid, block, 0, st, x, k, kp, q_nat,
                           q_perm, s, sumq);
}

hipError_t launch_act_quant(const void *x, bool bf16, int64_t m, int64_t k, int64_t kp, int8_t *q_nat,
                            int8_t *q_perm, float *s, int32_t *sumq, hipStream_t st)
{
    const bool full = k % 16 == 0;
    if (bf16) {
        const bf16_t *xb = static_cast<const bf16_t *>(x);
        if (full) launch_rg<bf16_t, true>(xb, m, k, kp, q_nat, q_perm, s, sumq, st);
        else launch_rg<bf16_t, false>(xb, m, k, kp, q_nat, q_perm, s, sumq, st);
    } else {
        const float *xf = static_cast<const float *>(x);
        if (full) launch_rg<float, true>(xf, m, k, kp, q_nat, q_perm, s, sumq, st);
        else launch_rg<float, false>(xf, m, k, kp, q_nat, q_perm, s, sumq, st);
    }
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
