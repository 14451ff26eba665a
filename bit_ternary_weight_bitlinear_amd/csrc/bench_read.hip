// bench_read.hip -- plain streaming reads of a packed weight matrix, the
// achievable-bandwidth ceiling the decode kernel is measured against.
//
// Measurement only: built into its own library (libbitlinear_bench.so), loaded
// by the benchmark, never by the product path. A launch reads one matrix of
// `rows` rows of `ldw` bytes (ldw % 16 == 0) with 16-byte non-temporal loads,
// every load of a thread issued before any is consumed, and folds the words
// into one XOR per thread; a thread writes it to sink[workgroup] only if it
// equals `key`, a run-time value the compiler cannot see through (so the loads
// stay); with a random key that store practically never happens.
//
// Two access patterns:
//  ROWS   -- the decode kernel's: workgroup b owns rows [b*R, b*R + R); a row is
//            cut into 128-byte pieces (eight 16-byte chunks), a group of 8 lanes
//            takes one (row, piece) unit and each lane one chunk, units go to the
//            groups row index fastest;
//  LINEAR -- the matrix as one flat array, workgroup b owns bytes/grid
//            contiguous bytes and a wave reads 1 KB contiguous per load.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ inline uint32_t load_fold(const uint8_t *p)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return v.x ^ v.y ^ v.z ^ v.w;
}

template <int JM>
__global__ __launch_bounds__(512) void read_rows_kernel(const uint8_t *src, int64_t rows, int64_t ldw, int R,
                                                        uint32_t key, uint32_t *sink)
{
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int64_t r0 = (int64_t)blockIdx.x * R;
    const int my_rows = (int)((rows - r0) < R ? (rows - r0) : R);
    const int C = (int)(ldw / 16);             // 16-byte chunks per row
    const int pieces = (C + 7) / 8;            // 128-byte pieces per row
    const int nunit = my_rows * pieces;
    const int grp = tid >> 3, li = tid & 7, ngrp = nthreads >> 3;
    uint32_t acc = 0;
    uint32_t v[JM];
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        int u = grp + j * ngrp;
        u = u < nunit ? u : nunit - 1;
        const int r = u % my_rows, b = u / my_rows;
        int c = 8 * b + li;
        c = c < C ? c : C - 1;
        v[j] = load_fold(src + (r0 + r) * ldw + (int64_t)c * 16);
    }
#pragma unroll
    for (int j = 0; j < JM; ++j) acc ^= v[j];
    if (acc == key) sink[blockIdx.x] = acc;
}

template <int JM>
__global__ __launch_bounds__(512) void read_linear_kernel(const uint8_t *src, int64_t bytes, uint32_t key,
                                                          uint32_t *sink)
{
    const int64_t per_wg = bytes / gridDim.x;  // multiple of 16 (checked on the host)
    const uint8_t *base = src + (int64_t)blockIdx.x * per_wg;
    const int64_t words = per_wg / 16;
    uint32_t acc = 0;
    uint32_t v[JM];
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        int64_t w = threadIdx.x + (int64_t)j * blockDim.x;
        w = w < words ? w : words - 1;
        v[j] = load_fold(base + w * 16);
    }
#pragma unroll
    for (int j = 0; j < JM; ++j) acc ^= v[j];
    if (acc == key) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads rows x ldw bytes in the decode kernel's pattern: `grid` workgroups of
// `threads` threads (64..512, a multiple of 64), R = ceil(rows / grid) rows each.
// sink: device uint32 [>= grid]. Returns 0, or -1 for arguments the kernel does
// not support (checked here), -2 if the launch fails.
int blbench_read_rows(const void *src, int64_t rows, int64_t ldw, int grid, int threads, uint32_t key,
                      uint32_t *sink, void *stream)
{
    if (!src || !sink || rows < 1 || ldw < 16 || ldw % 16 || grid < 1 || grid > 65536 || threads < 64 ||
        threads > 512 || threads % 64)
        return -1;
    const int64_t R = (rows + grid - 1) / grid;
    const int64_t units = R * ((ldw / 16 + 7) / 8);
    const int64_t jm = (units + threads / 8 - 1) / (threads / 8);
    const dim3 g((unsigned)((rows + R - 1) / R)), b((unsigned)threads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (jm <= 4) hipLaunchKernelGGL(read_rows_kernel<4>, g, b, 0, st, (const uint8_t *)src, rows, ldw, (int)R, key, sink);
    else if (jm <= 8) hipLaunchKernelGGL(read_rows_kernel<8>, g, b, 0, st, (const uint8_t *)src, rows, ldw, (int)R, key, sink);
    else if (jm <= 16) hipLaunchKernelGGL(read_rows_kernel<16>, g, b, 0, st, (const uint8_t *)src, rows, ldw, (int)R, key, sink);
    else return -1;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Reads `bytes` (a multiple of 16 * grid) as one flat array: `grid` workgroups
// of `threads` threads, each workgroup a contiguous bytes/grid block.
// sink: device uint32 [>= grid].
int blbench_read_linear(const void *src, int64_t bytes, int grid, int threads, uint32_t key, uint32_t *sink,
                        void *stream)
{
    if (!src || !sink || bytes < 16 || grid < 1 || grid > 65536 || bytes % (16 * (int64_t)grid) ||
        threads < 64 || threads > 512 || threads % 64)
        return -1;
    const int64_t words = bytes / grid / 16;
    const int64_t jm = (words + threads - 1) / threads;
    const dim3 g((unsigned)grid), b((unsigned)threads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (jm <= 2) hipLaunchKernelGGL(read_linear_kernel<2>, g, b, 0, st, (const uint8_t *)src, bytes, key, sink);
    else if (jm <= 4) hipLaunchKernelGGL(read_linear_kernel<4>, g, b, 0, st, (const uint8_t *)src, bytes, key, sink);
    else if (jm <= 8) hipLaunchKernelGGL(read_linear_kernel<8>, g, b, 0, st, (const uint8_t *)src, bytes, key, sink);
    else if (jm <= 16) hipLaunchKernelGGL(read_linear_kernel<16>, g, b, 0, st, (const uint8_t *)src, bytes, key, sink);
    else return -1;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
