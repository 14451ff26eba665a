// skinny.hip -- BitLinear for 5..64 tokens (batched decode) on gfx950.
//
// At a few dozen tokens the W1.58A8 product ("穿越1比特的奇幻旅程", section
// 推理实现 / GPU端) is still a stream over the packed weights, but too many
// tokens for v_dot4. It runs on v_mfma_i32_16x16x64_i8 with the weights as the
// A operand straight from HBM (no LDS staging: no two waves share a weight row):
//  * a workgroup owns 16 weight rows; its 4 waves split k in blocks of 256
//    inputs (four 64-input chunks), so ceil(n/16) workgroups cover the chip;
//  * per block, lane l loads 16 packed bytes = chunk (4b + l/16) of row l%16
//    and feeds dword s of it to MFMA s (s = 0..3): after the in-register 2-bit
//    expansion, dword s holds the codes of inputs 16s..16s+15 of that chunk in
//    the qperm byte order, matched by a 16-byte load of the qperm activations;
//  * the four waves' partial sums meet in LDS; the epilogue subtracts
//    sum_k q, rescales and stores.
// All sums are exact integers, so the split over waves does not change results.
// bitlinear_forward takes the kernel in bgemv.hip for these token counts when
// k <= 8192; this one serves longer rows, the FFN block's contractions and the
// integer-only entry point.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kSkRows = 16;

struct SkinnyArgs {
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
    float qmax;
};

// MB: 16-token blocks (1..4). EPI as for the GEMM. KB > 0: each wave has at
// most KB blocks, all requested at the start.
template <int MB, int EPI, int KB = 0>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs a)
{
    constexpr bool DUAL = EPI == EPI_GATE;
    constexpr int NA = DUAL ? 2 : 1;
    __shared__ int part[4][NA][MB][4][64];  // [wave][matrix][token block][reg][lane]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lh = lane >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * kSkRows;
    const int64_t row = (r0 + lr) < a.n ? (r0 + lr) : (a.n - 1);  // clamped; extra rows dropped
    const int chunks = (int)(a.kp / 64);
    const int nblk = (chunks + 3) / 4;

    v4i acc[NA][MB];
#pragma unroll
    for (int mat = 0; mat < NA; ++mat)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mat][mb] = v4i{0, 0, 0, 0};

    const uint8_t *wrow0 = a.w0 + row * a.ldw;
    const uint8_t *wrow1 = (DUAL ? a.w1 : a.w0) + row * a.ldw;

    // the epilogue's operands, requested before the weights: read after the
    // barrier they put an L2 round trip in front of the stores. Wave w's
    // epilogue covers token block w (MB <= 4), token 16 w + lane % 16.
    static_assert(MB <= 4, "one token block per wave in the epilogue");
    const int64_t me = wave * 16 + lr;
    int e_sq = 0;
    float e_s = 0.0f;
    if (wave < MB && me < a.m) {
        e_sq = a.sumq[me];
        if constexpr (EPI != EPI_ACC) e_s = a.s[me];
    }
    const float g0 = EPI != EPI_ACC ? a.gamma0[0] : 0.0f;
    const float g1 = DUAL ? a.gamma1[0] : 0.0f;

    // two blocks in flight per wave: loads of block b+4 are issued before block b is used
    auto load_block = [&](int b, v4u wv[NA], v4i qv[4][MB]) {
        const int c = 4 * b + lh;
        const bool ok = c < chunks;
        const int cc = ok ? c : chunks - 1;
#pragma unroll
        for (int mat = 0; mat < NA; ++mat) {
            const v4u w = __builtin_nontemporal_load(reinterpret_cast<const v4u *>((mat ? wrow1 : wrow0) + cc * 16));
            wv[mat] = ok ? w : v4u{0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int64_t tok = mb * 16 + lr;  // rows up to the padded token count exist
                const v4i q = *reinterpret_cast<const v4i *>(a.qp + tok * a.kp + cc * 64 + s * 16);
                qv[s][mb] = ok ? q : v4i{0, 0, 0, 0};
            }
    };

    if constexpr (KB > 0) {
        // every packed-weight block of this wave requested up front (KB of them,
        // blocks past the end are code 1 against zero activations); the
        // activations of block i+1 are loaded while block i runs
        v4u wv[KB][NA];
        v4i qa[4][MB], qb[4][MB];
#pragma unroll
        for (int i = 0; i < KB; ++i) load_block(wave + 4 * i, wv[i], i == 0 ? qa : qb);
        __builtin_amdgcn_sched_barrier(0);  // keep every request ahead of the first use
        asm volatile("" ::"s"(g0), "s"(g1));  // gamma fetched by now, not sunk to the epilogue
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            v4i (&qc)[4][MB] = (i & 1) ? qb : qa;
            v4i (&qn)[4][MB] = (i & 1) ? qa : qb;
            if (i + 1 < KB) {
                v4u unused[NA];
                load_block(wave + 4 * (i + 1), unused, qn);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int mat = 0; mat < NA; ++mat) {
                    const v4i av = expand_codes4(wv[i][mat][s]);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mat][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, qc[s][mb], acc[mat][mb], 0, 0, 0);
                }
        }
    } else {
    v4u wcur[NA], wnxt[NA];
    v4i qcur[4][MB], qnxt[4][MB];
    int b = wave;
    if (b < nblk) load_block(b, wcur, qcur);
    asm volatile("" ::"s"(g0), "s"(g1));  // gamma fetched by now, not sunk to the epilogue
    while (b < nblk) {
        const int bn = b + 4;
        if (bn < nblk) load_block(bn, wnxt, qnxt);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int mat = 0; mat < NA; ++mat) {
                const v4i av = expand_codes4(wcur[mat][s]);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mat][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, qcur[s][mb], acc[mat][mb], 0, 0, 0);
            }
        }
        b = bn;
#pragma unroll
        for (int mat = 0; mat < NA; ++mat) wcur[mat] = wnxt[mat];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) qcur[s][mb] = qnxt[s][mb];
    }
    }

    // combine the four waves' partial sums
#pragma unroll
    for (int mat = 0; mat < NA; ++mat)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 4; ++v) part[wave][mat][mb][v][lane] = acc[mat][mb][v];
    __syncthreads();

    // epilogue: thread -> (token block mb = wave, lane, reg v); C[n][m] with
    // n = 4*(lane/16) + v, m = lane%16
    for (int mb = wave; mb < MB; mb += 4) {
        const int64_t m = mb * 16 + lr;
        if (m >= a.m) continue;
        const int sq = e_sq;  // mb == wave
        float c0 = 0.0f, c1 = 0.0f;
        if constexpr (EPI != EPI_ACC) {
            c0 = token_scale(e_s, g0, a.qmax);
            if constexpr (DUAL) c1 = token_scale(e_s, g1, a.qmax);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t n = r0 + 4 * lh + v;
            if (n >= a.n) continue;
            int va = -sq, vb = -sq;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                va += part[w][0][mb][v][lane];
                if constexpr (DUAL) vb += part[w][NA - 1][mb][v][lane];
            }
            if constexpr (EPI == EPI_ACC) {
                a.acc_out[m * a.n + n] = va;
            } else if constexpr (DUAL) {
                a.out[m * a.n + n] = sq_relu_gate((float)va * c0, (float)vb * c1);
            } else {
                a.out[m * a.n + n] = (float)va * c0;
                if (a.acc_out) a.acc_out[m * a.n + n] = va;
            }
        }
    }
}

bool skinny_supported(int64_t m) { return m >= 1 && m <= 64; }

template <int MB, int KB = 0>
static void launch_mb(const SkinnyArgs &a, int epi, hipStream_t st)
{
    const dim3 grid((unsigned)ceil_div(a.n, kSkRows));
    switch (epi) {
    case EPI_Y: hipLaunchKernelGGL((skinny_kernel<MB, EPI_Y, KB>), grid, dim3(kThreads), 0, st, a); break;
    case EPI_ACC: hipLaunchKernelGGL((skinny_kernel<MB, EPI_ACC, KB>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((skinny_kernel<MB, EPI_GATE, KB>), grid, dim3(kThreads), 0, st, a); break;
    }
}

// up to 16 tokens: each wave's blocks (ceil(blocks / 4) of them) requested at once
static void launch_mb1(const SkinnyArgs &a, int epi, hipStream_t st)
{
    const int kb = (int)ceil_div(ceil_div(a.kp / 64, 4), 4);
    switch (kb) {
    case 1: launch_mb<1, 1>(a, epi, st); break;
    case 2: launch_mb<1, 2>(a, epi, st); break;
    case 3: launch_mb<1, 3>(a, epi, st); break;
    case 4: launch_mb<1, 4>(a, epi, st); break;
    case 5: launch_mb<1, 5>(a, epi, st); break;
    case 6: launch_mb<1, 6>(a, epi, st); break;
    case 7: launch_mb<1, 7>(a, epi, st); break;
    case 8: launch_mb<1, 8>(a, epi, st); break;
    default: launch_mb<1>(a, epi, st); break;
    }
}

hipError_t launch_skinny(const GemmProblem &p, hipStream_t st)
{
    SkinnyArgs a;
    a.qp = p.qp; a.kp = p.kp; a.s = p.s; a.sumq = p.sumq; a.m = p.m; a.n = p.n;
    a.w0 = p.w0; a.w1 = p.w1; a.ldw = p.ldw; a.gamma0 = p.gamma0; a.gamma1 = p.gamma1;
    a.out = p.out; a.acc_out = p.acc_out; a.qmax = p.qmax;
    switch ((p.m + 15) / 16) {
    case 1: launch_mb1(a, p.epi, st); break;
    case 2: launch_mb<2>(a, p.epi, st); break;
    case 3: launch_mb<3>(a, p.epi, st); break;
    default: launch_mb<4>(a, p.epi, st); break;
    }
    return hipGetLastError();
}

}  // namespace bl
