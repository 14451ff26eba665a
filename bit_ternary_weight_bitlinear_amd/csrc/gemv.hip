// gemv.hip -- decode-time BitLinear (m <= 4 tokens) for gfx950.
//
// The W1.58A8 product ("穿越1比特的奇幻旅程", section 推理实现 / GPU端) at small m is a
// stream over the packed weights: 2 bits per weight is the whole HBM traffic,
// so the kernel is built to keep every CU's loads in flight:
//  * each thread first issues all of its 16-byte non-temporal loads of packed
//    weights (up to 8 per matrix), before doing anything else;
//  * while they are in flight, the workgroup quantizes the m tokens itself
//    (absmax with DPP wave reductions, then rint) into LDS in the qperm order,
//    so there is no separate activation kernel and no launch gap;
//  * the codes are decoded in registers with four AND masks and one shift per
//    dword (code<<0, <<2, <<4 and, after a right shift by one, <<5 -- all fit in
//    a signed byte) and fed to v_dot4_i32_i8 against the qperm dwords; the
//    four partial sums are rescaled by exact shifts at the end;
//  * a row is split over `lpr` lanes (a power of two), reduced with lane shuffles.
// Integer sums are exact, so the result is independent of the lane split.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kMaxChunks = 8;       // 16-byte chunks per thread and matrix
constexpr int kGemvLdsLimit = 60 * 1024;

struct GemvArgs {
    const void *x;
    int64_t k, kp, n;
    const uint8_t *w0, *w1;
    int64_t ldw;
    const float *gamma0, *gamma1;
    float *out;
    int32_t *acc_out;
    int8_t *q_out;
    float *s_out;
    int lpr_log2, nch, chunks;
};

// LDS slot of group (c, d): 16-byte slots rotated by (c >> 2) & 3 so that the
// lanes of one row, which read neighbouring chunks, spread over the banks.
__device__ inline int lds_slot(int c, int d) { return c * 64 + ((d ^ ((c >> 2) & 3)) << 4); }

template <typename T, bool VEC, int MT, bool DUAL>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a)
{
    extern __shared__ __align__(16) int8_t q_lds[];  // [MT][kp]
    __shared__ float red_f[MT][4];
    __shared__ int red_i[MT][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lpr = 1 << a.lpr_log2;
    const int p = tid & (lpr - 1);
    const int64_t row = (int64_t)blockIdx.x * (kThreads >> a.lpr_log2) + (tid >> a.lpr_log2);
    const bool row_ok = row < a.n;

    // 1. issue every packed-weight load of this thread
    uint4 wa[kMaxChunks], wb[kMaxChunks];
    {
        const uint4 *pa = reinterpret_cast<const uint4 *>(a.w0 + (row_ok ? row : 0) * a.ldw);
        const uint4 *pb = reinterpret_cast<const uint4 *>((DUAL ? a.w1 : a.w0) + (row_ok ? row : 0) * a.ldw);
#pragma unroll
        for (int j = 0; j < kMaxChunks; ++j) {
            const int c = p + (j << a.lpr_log2);
            const bool ok = row_ok && j < a.nch && c < a.chunks;
            wa[j] = ok ? load_nt16(pa + c) : make_uint4(0, 0, 0, 0);
            if constexpr (DUAL) wb[j] = ok ? load_nt16(pb + c) : make_uint4(0, 0, 0, 0);
        }
    }

    // 2. per-token absmax quantization of the MT tokens into LDS
    const T *x = static_cast<const T *>(a.x);
    const int64_t G = ceil_div(a.k, 16);
    const int GP = (int)(a.kp / 16);
    float st[MT], inv[MT];
    int sq[MT];
    {
        float amax[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            amax[t] = 0.0f;
            for (int64_t g = tid; g < G; g += kThreads) {
                float f[16];
                load_group<T, VEC>(x + t * a.k, a.k, g, f);
#pragma unroll
                for (int j = 0; j < 16; ++j) amax[t] = fmaxf(amax[t], fabsf(f[j]));
            }
            amax[t] = wave_max(amax[t]);
            if (lane == 0) red_f[t][wave] = amax[t];
        }
        __syncthreads();
        int qs[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            st[t] = fmaxf(fmaxf(fmaxf(red_f[t][0], red_f[t][1]), fmaxf(red_f[t][2], red_f[t][3])), kEps);
            inv[t] = 127.0f / st[t];
            qs[t] = 0;
            for (int g = tid; g < GP; g += kThreads) {
                float f[16];
                if (g < G) {
                    load_group<T, VEC>(x + t * a.k, a.k, g, f);
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j) f[j] = 0.0f;
                }
                int qi[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    qi[j] = quant_i8(f[j], inv[t]);
                    qs[t] += qi[j];
                }
                const int c = g >> 2, d = g & 3;
                *reinterpret_cast<uint4 *>(q_lds + t * a.kp + lds_slot(c, d)) = qperm_pack(qi);
                if (a.q_out && blockIdx.x == 0 && g < G) {
                    const uint4 v = qnat_pack(qi);
                    const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
                    uint32_t *dst = reinterpret_cast<uint32_t *>(a.q_out + t * a.k + 16 * (int64_t)g);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (16 * (int64_t)g + 4 * j < a.k) dst[j] = dw[j];
                }
            }
            qs[t] = wave_sum(qs[t]);
            if (lane == 0) red_i[t][wave] = qs[t];
            if (a.s_out && blockIdx.x == 0 && tid == 0) a.s_out[t] = st[t];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < MT; ++t) sq[t] = red_i[t][0] + red_i[t][1] + red_i[t][2] + red_i[t][3];
    }

    // 3. decode the 2-bit codes in registers, v_dot4 against the qperm dwords
    int acc[MT][4], accb[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = accb[t][i] = 0;

#pragma unroll
    for (int j = 0; j < kMaxChunks; ++j) {
        const int c = p + (j << a.lpr_log2);
        if (j < a.nch && c < a.chunks) {
            const uint32_t wda[4] = {wa[j].x, wa[j].y, wa[j].z, wa[j].w};
            const uint32_t wdb[4] = {wb[j].x, wb[j].y, wb[j].z, wb[j].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int e0 = (int)(wda[d] & 0x03030303u);
                const int e1 = (int)(wda[d] & 0x0C0C0C0Cu);
                const int e2 = (int)(wda[d] & 0x30303030u);
                const int e3 = (int)((wda[d] >> 1) & 0x60606060u);
                int f0 = 0, f1 = 0, f2 = 0, f3 = 0;
                if constexpr (DUAL) {
                    f0 = (int)(wdb[d] & 0x03030303u);
                    f1 = (int)(wdb[d] & 0x0C0C0C0Cu);
                    f2 = (int)(wdb[d] & 0x30303030u);
                    f3 = (int)((wdb[d] >> 1) & 0x60606060u);
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const v4i qv = *reinterpret_cast<const v4i *>(q_lds + t * a.kp + lds_slot(c, d));
                    acc[t][0] = __builtin_amdgcn_sdot4(e0, qv.x, acc[t][0], false);
                    acc[t][1] = __builtin_amdgcn_sdot4(e1, qv.y, acc[t][1], false);
                    acc[t][2] = __builtin_amdgcn_sdot4(e2, qv.z, acc[t][2], false);
                    acc[t][3] = __builtin_amdgcn_sdot4(e3, qv.w, acc[t][3], false);
                    if constexpr (DUAL) {
                        accb[t][0] = __builtin_amdgcn_sdot4(f0, qv.x, accb[t][0], false);
                        accb[t][1] = __builtin_amdgcn_sdot4(f1, qv.y, accb[t][1], false);
                        accb[t][2] = __builtin_amdgcn_sdot4(f2, qv.z, accb[t][2], false);
                        accb[t][3] = __builtin_amdgcn_sdot4(f3, qv.w, accb[t][3], false);
                    }
                }
            }
        }
    }

    // 4. undo the field shifts, reduce over the lanes of the row, rescale
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int ta = acc[t][0] + (acc[t][1] >> 2) + (acc[t][2] >> 4) + (acc[t][3] >> 5);
        int tb = accb[t][0] + (accb[t][1] >> 2) + (accb[t][2] >> 4) + (accb[t][3] >> 5);
        for (int off = lpr >> 1; off > 0; off >>= 1) {
            ta += __shfl_xor(ta, off);
            if constexpr (DUAL) tb += __shfl_xor(tb, off);
        }
        if (p == 0 && row_ok) {
            const int va = ta - sq[t];
            const float ya = (float)va * token_scale(st[t], a.gamma0[0]);
            if constexpr (DUAL) {
                const int vb = tb - sq[t];
                const float yb = (float)vb * token_scale(st[t], a.gamma1[0]);
                a.out[t * a.n + row] = sq_relu_gate(ya, yb);
            } else {
                a.out[t * a.n + row] = ya;
                if (a.acc_out) a.acc_out[t * a.n + row] = va;
            }
        }
    }
}

bool gemv_supported(int64_t m, int64_t kp)
{
    const int64_t chunks = kp / 64;
    return m >= 1 && m <= 4 && m * kp <= kGemvLdsLimit && chunks <= 64 * kMaxChunks;
}

template <typename T, bool VEC, bool DUAL>
static void launch_mt(int mt, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    switch (mt) {
    case 1: hipLaunchKernelGGL((gemv_kernel<T, VEC, 1, DUAL>), grid, dim3(kThreads), lds, st, a); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<T, VEC, 2, DUAL>), grid, dim3(kThreads), lds, st, a); break;
    case 3: hipLaunchKernelGGL((gemv_kernel<T, VEC, 3, DUAL>), grid, dim3(kThreads), lds, st, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<T, VEC, 4, DUAL>), grid, dim3(kThreads), lds, st, a); break;
    }
}

hipError_t launch_gemv(const GemvProblem &p, hipStream_t st)
{
    GemvArgs a;
    a.x = p.x; a.k = p.k; a.kp = p.kp; a.n = p.n;
    a.w0 = p.w0; a.w1 = p.w1; a.ldw = p.ldw;
    a.gamma0 = p.gamma0; a.gamma1 = p.gamma1;
    a.out = p.out; a.acc_out = p.acc_out; a.q_out = p.q_out; a.s_out = p.s_out;
    a.chunks = (int)(p.kp / 64);

    // lanes per row: the fewest that keep <= 8 chunks per lane, then more lanes
    // while the grid is smaller than the chip and the lanes stay >= 75 % busy
    int lg = 0;
    while (ceil_div(a.chunks, 1 << lg) > kMaxChunks) ++lg;
    while (lg < 6) {
        const int64_t blocks = ceil_div(p.n, kThreads >> lg);
        const int nlg = lg + 1;
        const int64_t nch2 = ceil_div(a.chunks, 1 << nlg);
        const double eff = (double)a.chunks / (double)(nch2 << nlg);
        if (blocks >= 256 || eff < 0.75) break;
        lg = nlg;
    }
    a.lpr_log2 = lg;
    a.nch = (int)ceil_div(a.chunks, 1 << lg);
    const dim3 grid((unsigned)ceil_div(p.n, kThreads >> lg));
    const size_t lds = (size_t)(p.m * p.kp);
    const bool dual = p.w1 != nullptr;
    if (p.bf16) {
        const bool vec = p.k % 8 == 0;
        if (dual) {
            if (vec) launch_mt<bf16_t, true, true>((int)p.m, grid, lds, st, a);
            else launch_mt<bf16_t, false, true>((int)p.m, grid, lds, st, a);
        } else {
            if (vec) launch_mt<bf16_t, true, false>((int)p.m, grid, lds, st, a);
            else launch_mt<bf16_t, false, false>((int)p.m, grid, lds, st, a);
        }
    } else {
        if (dual) launch_mt<float, true, true>((int)p.m, grid, lds, st, a);
        else launch_mt<float, true, false>((int)p.m, grid, lds, st, a);
    }
    return hipGetLastError();
}

}  // namespace bl
