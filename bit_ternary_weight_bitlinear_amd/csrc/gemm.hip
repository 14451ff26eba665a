// gemm.hip -- BitLinear at m > 4 tokens on the gfx950 int8 matrix cores.
//
// At many tokens the W1.58A8 product ("穿越1比特的奇幻旅程", section 推理实现 / GPU端)
// is a dense contraction, so it runs on v_mfma_i32_32x32x32_i8:
//  * A operand = weights. Each k-step, the workgroup loads its BN packed rows
//    (16 bytes = 64 weights per row), expands the 2-bit codes to int8 in
//    registers ((w >> 2i) & 0x03030303 gives the codes of inputs 16g+4b+i, i.e.
//    exactly the qperm byte order) and writes the int8 tile to LDS.
//  * B operand = qperm activations, copied to LDS as they are.
//  * Codes are w+1 in {0,1,2}; the epilogue subtracts sum_k q per token.
//  * C[n][m] per 32x32 block: lane l holds n = 8*(v/4) + 4*(l/32) + v%4 and
//    m = l%32, so every lane stores 4 consecutive outputs of one token (16 B).
// Integer accumulation is exact; the fp32 rescale matches the decode path bit
// for bit.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kLdsStride = 80;  // bytes per 64-byte tile row (16 bytes of padding)

struct GemmArgs {
    const int8_t *qp;
    int64_t kp;
    const float *s;
    const int32_t *sumq;
    int64_t m, n;
    const uint8_t *w0, *w1;
    int64_t ldw;
    const float *gamma0, *gamma1;
    float *out;
    int32_t *acc_out;
};

__device__ inline uint4 expand_codes(uint32_t w)
{
    return make_uint4(w & 0x03030303u, (w >> 2) & 0x03030303u, (w >> 4) & 0x03030303u,
                      (w >> 6) & 0x03030303u);
}

template <int BN, int BM, int WN, int WM, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a)
{
    constexpr bool DUAL = EPI == EPI_GATE;
    constexpr int NA = DUAL ? 2 : 1;
    constexpr int NWN = BN / WN, NWM = BM / WM;
    static_assert(NWN * NWM == 4, "four waves per workgroup");
    constexpr int FN = WN / 32, FM = WM / 32;
    constexpr int A_LD = (BN + kThreads - 1) / kThreads;
    constexpr int B_LD = (BM * 4 + kThreads - 1) / kThreads;

    __shared__ __align__(16) int8_t As[NA][BN * kLdsStride];
    __shared__ __align__(16) int8_t Bs[BM * kLdsStride];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % NWN, wm = wave / NWN;
    const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;

    uint4 ra[NA][A_LD], rb[B_LD];
    auto gload = [&](int64_t ks) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int r = tid + i * kThreads;
            const int64_t n = n0 + r;
            const bool ok = r < BN && n < a.n;
#pragma unroll
            for (int mat = 0; mat < NA; ++mat) {
                const uint8_t *w = mat == 0 ? a.w0 : a.w1;
                ra[mat][i] = ok ? *reinterpret_cast<const uint4 *>(w + n * a.ldw + ks * 16)
                                : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int e = tid + i * kThreads;
            if (e < BM * 4) {
                const int r = e >> 2, part = e & 3;
                rb[i] = *reinterpret_cast<const uint4 *>(a.qp + (m0 + r) * a.kp + ks * 64 + part * 16);
            }
        }
    };
    auto swrite = [&]() {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int r = tid + i * kThreads;
            if (r < BN) {
#pragma unroll
                for (int mat = 0; mat < NA; ++mat) {
                    const uint32_t wd[4] = {ra[mat][i].x, ra[mat][i].y, ra[mat][i].z, ra[mat][i].w};
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        *reinterpret_cast<uint4 *>(&As[mat][r * kLdsStride + d * 16]) = expand_codes(wd[d]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int e = tid + i * kThreads;
            if (e < BM * 4) {
                const int r = e >> 2, part = e & 3;
                *reinterpret_cast<uint4 *>(&Bs[r * kLdsStride + part * 16]) = rb[i];
            }
        }
    };

    v16i acc[NA][FN][FM];
#pragma unroll
    for (int mat = 0; mat < NA; ++mat)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mat][fn][fm][v] = 0;

    const int64_t nks = a.kp / 64;
    gload(0);
    for (int64_t ks = 0; ks < nks; ++ks) {
        __syncthreads();
        swrite();
        __syncthreads();
        if (ks + 1 < nks) gload(ks + 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int col = (2 * s + (lane >> 5)) * 16;
            v4i bf[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                bf[fm] = *reinterpret_cast<const v4i *>(&Bs[(wm * WM + fm * 32 + (lane & 31)) * kLdsStride + col]);
#pragma unroll
            for (int mat = 0; mat < NA; ++mat)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const v4i af = *reinterpret_cast<const v4i *>(
                        &As[mat][(wn * WN + fn * 32 + (lane & 31)) * kLdsStride + col]);
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
                        acc[mat][fn][fm] =
                            __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf[fm], acc[mat][fn][fm], 0, 0, 0);
                }
        }
    }

    // epilogue
    const bool vec_ok = (a.n % 4) == 0;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int64_t m = m0 + wm * WM + fm * 32 + (lane & 31);
        if (m >= a.m) continue;
        const int sq = a.sumq[m];
        float c0 = 0.0f, c1 = 0.0f;  // the integer-only epilogue has no scales
        if constexpr (EPI != EPI_ACC) {
            const float s = a.s[m];
            c0 = token_scale(s, a.gamma0[0]);
            if constexpr (DUAL) c1 = token_scale(s, a.gamma1[0]);
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t n = n0 + wn * WN + fn * 32 + 8 * j + 4 * (lane >> 5);
                int va[4];
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    va[e] = acc[0][fn][fm][4 * j + e] - sq;
                    if constexpr (DUAL) {
                        const int vb = acc[NA - 1][fn][fm][4 * j + e] - sq;
                        o[e] = sq_relu_gate((float)va[e] * c0, (float)vb * c1);
                    } else {
                        o[e] = (float)va[e] * c0;
                    }
                }
                if (vec_ok && n + 3 < a.n) {
                    if constexpr (EPI != EPI_ACC)
                        *reinterpret_cast<float4 *>(a.out + m * a.n + n) = make_float4(o[0], o[1], o[2], o[3]);
                    if (EPI == EPI_ACC || (EPI == EPI_Y && a.acc_out))
                        *reinterpret_cast<int4 *>(a.acc_out + m * a.n + n) = make_int4(va[0], va[1], va[2], va[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (n + e < a.n) {
                            if constexpr (EPI != EPI_ACC) a.out[m * a.n + n + e] = o[e];
                            if (EPI == EPI_ACC || (EPI == EPI_Y && a.acc_out)) a.acc_out[m * a.n + n + e] = va[e];
                        }
                    }
                }
            }
    }
}

template <int BN, int BM, int WN, int WM>
static void launch_tile(const GemmArgs &a, int epi, hipStream_t st)
{
    const dim3 grid((unsigned)ceil_div(a.n, BN), (unsigned)ceil_div(a.m, BM));
    switch (epi) {
    case EPI_Y: hipLaunchKernelGGL((gemm_kernel<BN, BM, WN, WM, EPI_Y>), grid, dim3(kThreads), 0, st, a); break;
    case EPI_ACC: hipLaunchKernelGGL((gemm_kernel<BN, BM, WN, WM, EPI_ACC>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((gemm_kernel<BN, BM, WN, WM, EPI_GATE>), grid, dim3(kThreads), 0, st, a); break;
    }
}

hipError_t launch_gemm(const GemmProblem &p, hipStream_t st)
{
    GemmArgs a;
    a.qp = p.qp; a.kp = p.kp; a.s = p.s; a.sumq = p.sumq; a.m = p.m; a.n = p.n;
    a.w0 = p.w0; a.w1 = p.w1; a.ldw = p.ldw; a.gamma0 = p.gamma0; a.gamma1 = p.gamma1;
    a.out = p.out; a.acc_out = p.acc_out;
    if (p.m <= 32)
        launch_tile<256, 32, 64, 32>(a, p.epi, st);
    else if (p.m <= 64)
        launch_tile<256, 64, 64, 64>(a, p.epi, st);
    else
        launch_tile<128, 128, 64, 64>(a, p.epi, st);
    return hipGetLastError();
}

}  // namespace bl
