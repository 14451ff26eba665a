// pack.hip -- offline absmean ternarization and 2-bit packing for gfx950.
//
// Weight quantizer: gamma = mean|W| over the tensor, W~ = clip(rint(W / gamma), -1, 1)
// ("BitNet 1-bit LLM 的混合精度微调技术", BitLinear and operational-parameter
// paragraphs; "穿越1比特的奇幻旅程", section 架构创新), stored as the code w+1, four
// per byte ("穿越1比特的奇幻旅程", section 推理实现 / GPU端).
//
// The mean is accumulated in fp64 in one fixed order -- each row left to right,
// then the row sums in row order -- so gamma is the same bits on every run and
// every device. The codes then depend on a correctly rounded fp32 division.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

// One wave per 64 rows. 64x64 tiles of W are staged through LDS so that the
// global reads are coalesced while each lane walks its own row in k order.
__global__ __launch_bounds__(64) void absmean_rowsum_kernel(const float *__restrict__ w, int64_t n,
                                                            int64_t k, double *__restrict__ rowsum)
{
    __shared__ float tile[64][65];
    const int lane = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    double acc = 0.0;
    for (int64_t c0 = 0; c0 < k; c0 += 64) {
        const int64_t c = c0 + lane;
#pragma unroll 8
        for (int i = 0; i < 64; ++i) {
            const int64_t r = r0 + i;
            tile[i][lane] = (r < n && c < k) ? w[r * k + c] : 0.0f;
        }
        __syncthreads();
        const int cnt = (int)((k - c0) < 64 ? (k - c0) : 64);
        for (int j = 0; j < cnt; ++j) acc += fabs((double)tile[lane][j]);
        __syncthreads();
    }
    if (r0 + lane < n) rowsum[r0 + lane] = acc;
}

// Sequential sum of the row sums (row order), one division, one rounding to fp32.
__global__ void absmean_finish_kernel(const double *__restrict__ rowsum, int64_t n, int64_t k,
                                      float *__restrict__ gamma)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    double total = 0.0;
    for (int64_t r = 0; r < n; ++r) total += rowsum[r];
    gamma[0] = (float)(total / ((double)n * (double)k));
}

// One packed byte per thread (four weights, one 16-byte load).
__global__ __launch_bounds__(256) void ternary_pack_kernel(const float *__restrict__ w, int64_t n,
                                                           int64_t k, const float *__restrict__ gamma,
                                                           uint8_t *__restrict__ packed)
{
    const int64_t kb = k / 4;
    const int64_t total = n * kb;
    const float g = gamma[0];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / kb, j = i - r * kb;
        const float4 v = *reinterpret_cast<const float4 *>(w + r * k + 4 * j);
        const float e[4] = {v.x, v.y, v.z, v.w};
        uint32_t byte = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float q = (g > 0.0f) ? e[t] / g : 0.0f;
            q = __builtin_rintf(q);
            q = fminf(fmaxf(q, -1.0f), 1.0f);
            byte |= (uint32_t)((int)q + 1) << (2 * t);
        }
        packed[i] = (uint8_t)byte;
    }
}

hipError_t launch_pack(const float *w, int64_t n, int64_t k, uint8_t *packed, float *gamma,
                       double *rowsum, hipStream_t st)
{
    hipLaunchKernelGGL(absmean_rowsum_kernel, dim3((unsigned)ceil_div(n, 64)), dim3(64), 0, st, w, n,
                       k, rowsum);
    hipLaunchKernelGGL(absmean_finish_kernel, dim3(1), dim3(64), 0, st, rowsum, n, k, gamma);
    const int64_t total = n * (k / 4);
    int64_t blocks = ceil_div(total, 256);
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(ternary_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, w, n, k, gamma,
                       packed);
    return hipGetLastError();
}

// Row-wise copy into a padded stride; the tail bytes hold code 1 (weight 0).
__global__ __launch_bounds__(256) void pad_weights_kernel(const uint8_t *__restrict__ src, int64_t n,
                                                          int64_t kb, int64_t kpb,
                                                          uint8_t *__restrict__ dst)
{
    const int64_t total = n * kpb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / kpb, j = i - r * kpb;
        dst[i] = j < kb ? src[r * kb + j] : (uint8_t)0x55;
    }
}

hipError_t launch_pad_weights(const uint8_t *src, int64_t n, int64_t k, int64_t kp, uint8_t *dst,
                              hipStream_t st)
{
    const int64_t total = n * (kp / 4);
    int64_t blocks = ceil_div(total, 256);
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(pad_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, n, k / 4,
                       kp / 4, dst);
    return hipGetLastError();
}

}  // namespace bl
