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
//
// Threshold quantizer ("BitNet 三元权重阈值优化工程实践", section on the core
// principle of ternary threshold optimization): delta = factor * mean|W| (fp32
// product), w~ = sign(w) where |w| > delta (strict), else 0, and the scale alpha
// = the mean over all n*k weights of |w| times that mask, summed in the same
// fixed fp64 order. Same packed layout; alpha takes gamma's place downstream.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

// One thread per row: each row is one sequential fp64 chain (the order the
// definition fixes), so the parallelism is across rows. A lane keeps two
// batches of its row in flight (16 independent 16-byte loads each) and adds
// the current one in column order while the next arrives; a wave's 64 rows
// share each cache line over four consecutive loads.
// MASKED: only magnitudes above delta[0] count; the others add +0.0, which
// leaves an fp64 sum unchanged, so the sum equals the plain conditional one.
template <bool MASKED>
__global__ __launch_bounds__(64) void absmean_rowsum_kernel(const float *__restrict__ w, int64_t n,
                                                            int64_t k, const float *__restrict__ delta,
                                                            double *__restrict__ rowsum)
{
    constexpr int B = 16;  // float4 loads per batch (64 weights)
    const int64_t r = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (r >= n) return;
    const float *row = w + r * k;
    const int64_t nb = k / (4 * B);
    const float d = MASKED ? delta[0] : 0.0f;
    double acc = 0.0;
    auto mag = [&](float v) -> double {
        const float a = fabsf(v);
        if constexpr (MASKED) return a > d ? (double)a : 0.0;
        return (double)a;
    };
    auto add = [&](const float4 (&v)[B]) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            acc += mag(v[i].x);
            acc += mag(v[i].y);
            acc += mag(v[i].z);
            acc += mag(v[i].w);
        }
    };
    float4 cur[B], nxt[B];
    if (nb > 0) {
#pragma unroll
        for (int i = 0; i < B; ++i) cur[i] = *reinterpret_cast<const float4 *>(row + 4 * i);
    }
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t bn = b + 1 < nb ? b + 1 : b;  // the last batch re-reads itself (unused)
#pragma unroll
        for (int i = 0; i < B; ++i) nxt[i] = *reinterpret_cast<const float4 *>(row + bn * 4 * B + 4 * i);
        add(cur);
#pragma unroll
        for (int i = 0; i < B; ++i) cur[i] = nxt[i];
    }
    for (int64_t c = nb * 4 * B; c < k; ++c) acc += mag(row[c]);
    rowsum[r] = acc;
}

// Sequential sum of the row sums (row order), one division, one rounding to
// fp32. The workgroup stages the row sums in LDS with coalesced loads; thread 0
// adds them in order. DELTA: the result is multiplied by `factor` (one fp32
// product) -- the threshold delta rather than a scale.
template <bool DELTA>
__global__ __launch_bounds__(256) void absmean_finish_kernel(const double *__restrict__ rowsum, int64_t n,
                                                             int64_t k, float factor, float *__restrict__ gamma)
{
    constexpr int CH = 2048;
    __shared__ double buf[CH];
    double total = 0.0;
    for (int64_t base = 0; base < n; base += CH) {
        const int cnt = (int)((n - base) < CH ? (n - base) : CH);
        for (int i = threadIdx.x; i < cnt; i += blockDim.x) buf[i] = rowsum[base + i];
        __syncthreads();
        if (threadIdx.x == 0)
            for (int i = 0; i < cnt; ++i) total += buf[i];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const float mean = (float)(total / ((double)n * (double)k));
        gamma[0] = DELTA ? factor * mean : mean;
    }
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

// Threshold codes: one packed byte per thread.
__global__ __launch_bounds__(256) void threshold_pack_kernel(const float *__restrict__ w, int64_t n,
                                                             int64_t k, const float *__restrict__ delta,
                                                             uint8_t *__restrict__ packed)
{
    const int64_t kb = k / 4;
    const int64_t total = n * kb;
    const float d = delta[0];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / kb, j = i - r * kb;
        const float4 v = *reinterpret_cast<const float4 *>(w + r * k + 4 * j);
        const float e[4] = {v.x, v.y, v.z, v.w};
        uint32_t byte = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t code = fabsf(e[t]) > d ? (e[t] > 0.0f ? 2u : 0u) : 1u;
            byte |= code << (2 * t);
        }
        packed[i] = (uint8_t)byte;
    }
}

hipError_t launch_pack_threshold(const float *w, int64_t n, int64_t k, float factor, uint8_t *packed,
                                 float *alpha, float *delta, double *rowsum, hipStream_t st)
{
    const dim3 rows((unsigned)ceil_div(n, 64));
    hipLaunchKernelGGL(absmean_rowsum_kernel<false>, rows, dim3(64), 0, st, w, n, k, nullptr, rowsum);
    hipLaunchKernelGGL(absmean_finish_kernel<true>, dim3(1), dim3(256), 0, st, rowsum, n, k, factor, delta);
    hipLaunchKernelGGL(absmean_rowsum_kernel<true>, rows, dim3(64), 0, st, w, n, k, delta, rowsum);
    hipLaunchKernelGGL(absmean_finish_kernel<false>, dim3(1), dim3(256), 0, st, rowsum, n, k, 1.0f, alpha);
    const int64_t total = n * (k / 4);
    int64_t blocks = ceil_div(total, 256);
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(threshold_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, w, n, k, delta, packed);
    return hipGetLastError();
}

hipError_t launch_pack(const float *w, int64_t n, int64_t k, uint8_t *packed, float *gamma,
                       double *rowsum, hipStream_t st)
{
    hipLaunchKernelGGL(absmean_rowsum_kernel<false>, dim3((unsigned)ceil_div(n, 64)), dim3(64), 0, st, w, n,
                       k, nullptr, rowsum);
    hipLaunchKernelGGL(absmean_finish_kernel<false>, dim3(1), dim3(256), 0, st, rowsum, n, k, 1.0f, gamma);
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
