// bgemv.hip -- BitLinear for 5..16 tokens (batched decode) on gfx950, with the
// activation quantization inside the launch.
//
// The W1.58A8 product ("穿越1比特的奇幻旅程", section 推理实现 / GPU端) at a few
// tokens is still a stream over the packed weights. This kernel keeps the
// decode GEMV's structure -- one workgroup per CU owning a block of rows, all
// of its weight loads in flight at once, the tokens quantized by the
// workgroup itself -- and does the products on the int8 matrix cores:
//  * workgroup b owns rows [b*R, b*R + R), R = min(ceil(n / 256), 32), as one
//    or two 16-row blocks; with two blocks, even waves take block 0 and odd
//    waves block 1, and the waves of a block split k in quads of four 64-input
//    chunks;
//  * per quad, lane (h, r) = (lane / 16, lane % 16) loads the 16 packed bytes
//    of chunk 4*quad + h of row 16*block + r (rows past R re-read row R-1, so
//    the request merges with a valid lane's) and feeds dword s of it, expanded
//    in registers, as operand A of v_mfma_i32_16x16x64_i8 step s; operand B is
//    the 16 qperm bytes of token r at the same inputs, read from LDS;
//  * the m tokens (m*k up to 32768) are quantized once per workgroup, from
//    raw words loaded before the weights and converted after the weight loads
//    are issued: a per-token absmax (16-lane DPP maxima over the at most two
//    tokens a wave's 64 groups touch, merged by LDS atomics), one division per
//    token, then codes into LDS in qperm order (rows of whole chunk quads,
//    zero past k, plus 16 bytes: the 16 rows of one read phase fall on
//    different banks) and sum_k q per token. Larger m*k would cost every
//    workgroup too much arithmetic (2 us of VALU per CU at 8 x 6912 inputs);
//    there, the quantization kernel runs first and bmma.hip does the product;
//  * the waves' partial 16x16 blocks meet in LDS; the epilogue subtracts
//    sum_k q, rescales, stores y (and the int32 sums if asked).
// Integer sums are exact, so the split over waves and the order of the adds
// do not change results.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kBT = 512;       // threads per workgroup (8 waves)
constexpr int kBW = kBT / 64;  // waves per workgroup
constexpr int kBMaxTok = 16;   // tokens per launch: one 16-token MFMA block
constexpr int kBMaxRows = 32;  // at most two 16-row blocks per workgroup
constexpr int kBMaxK = 8192;

struct BgemvArgs {
    const void *x;  // bf16 / fp32 activations [m][k]
    int64_t m, k, kp, n;
    const uint8_t *w;
    int64_t ldw;
    const float *gamma;
    float *out;
    int32_t *acc_out;
    float qmax;
    int rows_per_wg;  // R
    int chunks;       // kp / 64
    uint32_t g_magic; // ceil(2^32 / (k / 16)): f / G as the high half of f * g_magic (exact for f * G < 2^32)
};

// RB: 16-row blocks per workgroup (1 or 2). JM: quads per wave. SL: activation
// groups of 16 inputs per thread (covering all m * k / 16 of them).
template <typename T, int RB, int JM, int SL>
__global__ __launch_bounds__(kBT) void bgemv_kernel(BgemvArgs a)
{
    extern __shared__ __align__(16) int8_t lds[];  // token rows [16][QS], then partial sums [kBW][4][64]
    __shared__ unsigned tok_max[kBMaxTok];
    __shared__ int tok_sum[kBMaxTok];
    __shared__ float tok_inv[kBMaxTok], tok_s[kBMaxTok];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lh = lane >> 4;
    const int M = (int)a.m;
    const int R = a.rows_per_wg, C = a.chunks;
    // LDS token rows: 16 of them, each 16 * GQ bytes of qperm codes (whole
    // quads of chunks; codes past kp and rows past the tokens are zero, so the
    // products read their operands without selects) plus 16 bytes, so the 16
    // rows of one read phase fall on different banks
    const int nq = (C + 3) >> 2;
    const int GQ = 16 * nq;
    const int QS = 16 * GQ + 16;
    int8_t *q_lds = lds;
    int *part = reinterpret_cast<int *>(lds + 16 * QS);
    const int64_t r0 = (int64_t)blockIdx.x * R;
    const int rows = (int)((a.n - r0) < R ? (a.n - r0) : R);
    const T *x = static_cast<const T *>(a.x);
    const int G = (int)(a.k / 16);  // k % 16 == 0
    const int NG = M * G;
    // gamma is requested now and waited for after the loads are out (fetched
    // in the epilogue it put an L2 round trip between the last barrier and
    // the stores)
    const float gam = a.gamma[0];

    if (tid < kBMaxTok) {
        tok_max[tid] = 0u;
        tok_sum[tid] = 0;
    }

    // 1. activation loads (raw words); slots no thread needs are not loaded
    //    (uniform). Slot s of a thread is the flat group f = tid + s * kBT,
    //    i.e. group f % G of token f / G; a token row is exactly G groups wide
    //    (k = 16 G), so its address is 16 f elements past the first row and
    //    the division waits until the loads are out
    constexpr int XQ = (int)sizeof(T);  // 16-byte words per group
    uint4 xq[SL][XQ];
    int slot_f[SL], slot_t[SL], slot_g[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
        slot_f[s] = min(tid + s * kBT, NG - 1);
        if (s * kBT < NG) {
            const uint4 *p = reinterpret_cast<const uint4 *>(x + 16 * (int64_t)slot_f[s]);
#pragma unroll
            for (int q = 0; q < XQ; ++q) xq[s][q] = p[q];
        } else {
#pragma unroll
            for (int q = 0; q < XQ; ++q) xq[s][q] = make_uint4(0, 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. weight quads of this wave: quad wave / RB + (kBW / RB) * j of row block
    //    wave % RB; slots past the last quad re-read the last one (dropped)
    const int rb = wave % RB;
    const int rr = min(16 * rb + lr, rows - 1);
    const uint8_t *wrow = a.w + (r0 + rr) * a.ldw;
    v4u wv[JM];
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        const int cq = min(wave / RB + (kBW / RB) * j, nq - 1);
        const int c = min(4 * cq + lh, C - 1);
        wv[j] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(wrow + c * 16));
        // issue order = use order, so each quad waits only for its own load
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::"s"(gam));
#pragma unroll
    for (int s = 0; s < SL; ++s) {
        slot_t[s] = (int)__umulhi((uint32_t)slot_f[s], a.g_magic);  // slot_f / G
        slot_g[s] = slot_f[s] - slot_t[s] * G;
    }

    // zero codes of each token's groups G .. GQ (their weight words are real
    // codes of a clamped chunk). The rows past the tokens are left as they are:
    // their products land in the columns of tokens the epilogue drops.
    for (int i = tid; i < M * (GQ - G); i += kBT) {
        const int t = i / (GQ - G), g = G + (i - t * (GQ - G));
        *reinterpret_cast<uint4 *>(q_lds + t * QS + g * 16) = make_uint4(0, 0, 0, 0);
    }

    // 3. per-token absmax. The 64 groups of one wave and slot belong to at most
    //    two tokens (u0 and u0 + 1: a token has G >= 64 groups); each 16-lane
    //    row reduces both with DPP and its lane 0 merges them into the tokens'
    //    maxima (integer max of non-negative float bits).
    __syncthreads();  // tok_max / tok_sum cleared
    float xk[SL][16];  // the inputs, converted once for both passes over them
#pragma unroll
    for (int s = 0; s < SL; ++s) {
        const int f0 = wave * 64 + s * kBT;  // first group of this wave and slot
        if (f0 >= NG) continue;              // uniform
        float *xr = xk[s];
        unpack_group<T>(xq[s], xr);
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(xr[j]));
        const bool valid = tid + s * kBT < NG;
        const int u0 = (int)__umulhi((uint32_t)f0, a.g_magic);  // f0 / G
        const float m0 = row16_max(valid && slot_t[s] == u0 ? mx : 0.0f);
        const float m1 = row16_max(valid && slot_t[s] != u0 ? mx : 0.0f);
        if (lr == 0) {
            atomicMax(&tok_max[u0], __float_as_uint(m0));
            if (u0 + 1 < M) atomicMax(&tok_max[u0 + 1], __float_as_uint(m1));
        }
    }
    __syncthreads();
    if (tid < M) {
        const float st = fmaxf(__uint_as_float(tok_max[tid]), kEps);
        tok_s[tid] = st;
        tok_inv[tid] = 127.0f / st;
    }
    __syncthreads();

    // 4. codes into LDS (qperm order) and sum_k q per token (inputs past k
    //    were zeroed above); the scales of every slot are read first, so the
    //    slots wait for LDS once
    float inv_s[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) inv_s[s] = tok_inv[slot_t[s]];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
        const int f0 = wave * 64 + s * kBT;
        if (f0 >= NG) continue;
        const bool valid = tid + s * kBT < NG;
        int sum = 0;
        if (valid) {
            uint4 pv;
            sum = quant_group(xk[s], inv_s[s], &pv, nullptr);
            *reinterpret_cast<uint4 *>(q_lds + slot_t[s] * QS + slot_g[s] * 16) = pv;
        }
        const int u0 = (int)__umulhi((uint32_t)f0, a.g_magic);  // f0 / G
        const int s0 = row16_sum(valid && slot_t[s] == u0 ? sum : 0);
        const int s1 = row16_sum(valid && slot_t[s] != u0 ? sum : 0);
        if (lr == 0) {
            atomicAdd(&tok_sum[u0], s0);
            if (u0 + 1 < M) atomicAdd(&tok_sum[u0 + 1], s1);
        }
    }
    __syncthreads();

    // 5. products: per quad, four MFMAs (dword s of each lane's 16 packed bytes
    //    against the qperm bytes of token lr at the same inputs); tokens past
    //    m and chunks past the row read zero codes
    v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        const int cq = wave / RB + (kBW / RB) * j;
        if (cq < nq) {  // uniform
            const int8_t *qc = q_lds + lr * QS + (4 * cq + lh) * 64;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(expand_codes4(wv[j][s]),
                                                             *reinterpret_cast<const v4i *>(qc + s * 16), acc, 0, 0, 0);
        }
    }
    // C[row][token]: lane (h, r) holds rows 4h + v (v = 0..3) of token r
#pragma unroll
    for (int v = 0; v < 4; ++v) part[(wave * 4 + v) * 64 + lane] = acc[v];
    __syncthreads();

    // 6. epilogue: item -> (row block, register v, lane), summed over the
    //    waves of its row block
    for (int e = tid; e < RB * 256; e += kBT) {
        const int eb = e >> 8, v = (e >> 6) & 3, el = e & 63;
        const int row = 16 * eb + 4 * (el >> 4) + v, t = el & 15;
        if (row < rows && t < M) {
            int va = -tok_sum[t];
#pragma unroll
            for (int w = eb; w < kBW; w += RB) va += part[(w * 4 + v) * 64 + el];
            const int64_t o = (int64_t)t * a.n + r0 + row;
            a.out[o] = (float)va * token_scale(tok_s[t], gam, a.qmax);
            if (a.acc_out) a.acc_out[o] = va;
        }
    }
}

// ---------------------------------------------------------------- host side

static int bgemv_slots(int64_t words) { return (int)ceil_div(words, (int64_t)kBT); }

// LDS bytes: 16 token rows of whole chunk quads plus 16 bytes, then the waves'
// partial sums
static size_t bgemv_lds(int64_t kp) { return (size_t)16 * (round_up(kp, 256) + 16) + (size_t)kBW * 4 * 64 * 4; }

bool bgemv_supported(int64_t m, int64_t k, bool bf16)
{
    // one token block, whole 16-input groups, at least 64 of them per token (a
    // wave's groups touch two tokens at most) and few enough inputs that
    // every workgroup may quantize them all
    return m >= 5 && m <= kBMaxTok && k <= kBMaxK && k % 16 == 0 && k >= 1024 && m * k <= 32768 &&
           bgemv_slots(m * k / 16) <= (bf16 ? 8 : 4);
}

namespace {

template <typename T, int RB, int JM, int SL>
hipError_t bg_launch(dim3 grid, size_t lds, hipStream_t st, const BgemvArgs &a)
{
    auto kern = bgemv_kernel<T, RB, JM, SL>;
    static LdsLimit lim;
    if (hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kern), (int)lds, lim)) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kBT), lds, st, a);
    return hipGetLastError();
}

template <typename T, int RB, int SL>
hipError_t bg_jm(int jm, dim3 grid, size_t lds, hipStream_t st, const BgemvArgs &a)
{
    if (jm <= 1) return bg_launch<T, RB, 1, SL>(grid, lds, st, a);
    if (jm <= 2) return bg_launch<T, RB, 2, SL>(grid, lds, st, a);
    if (jm <= 3) return bg_launch<T, RB, 3, SL>(grid, lds, st, a);
    if (jm <= 4) return bg_launch<T, RB, 4, SL>(grid, lds, st, a);
    if (jm <= 6) return bg_launch<T, RB, 6, SL>(grid, lds, st, a);
    return bg_launch<T, RB, 8, SL>(grid, lds, st, a);
}

template <typename T, int SL>
hipError_t bg_rb(int rb, int jm, dim3 grid, size_t lds, hipStream_t st, const BgemvArgs &a)
{
    return rb == 1 ? bg_jm<T, 1, SL>(jm, grid, lds, st, a) : bg_jm<T, 2, SL>(jm, grid, lds, st, a);
}

}  // namespace

hipError_t launch_bgemv(const GemvProblem &p, hipStream_t st)
{
    BgemvArgs a;
    a.x = p.x;
    a.m = p.m; a.k = p.k; a.kp = p.kp; a.n = p.n;
    a.w = p.w0; a.ldw = p.ldw; a.gamma = p.gamma0;
    a.out = p.out; a.acc_out = p.acc_out; a.qmax = p.qmax;
    a.chunks = (int)(p.kp / 64);
    a.g_magic = (uint32_t)ceil_div((int64_t)1 << 32, p.k / 16);
    int64_t r = ceil_div(p.n, (int64_t)256);
    if (r > kBMaxRows) r = kBMaxRows;
    a.rows_per_wg = (int)r;
    const int rb = r > 16 ? 2 : 1;
    const int64_t nq = ceil_div((int64_t)a.chunks, (int64_t)4);
    const int jm = (int)ceil_div(nq, (int64_t)(kBW / rb));  // <= 8: kp <= 8192
    const dim3 grid((unsigned)ceil_div(p.n, r));
    const size_t lds = bgemv_lds(p.kp);
    const int sl = bgemv_slots(p.m * p.k / 16);
    if (p.bf16) {
        if (sl <= 2) return bg_rb<bf16_t, 2>(rb, jm, grid, lds, st, a);
        if (sl <= 4) return bg_rb<bf16_t, 4>(rb, jm, grid, lds, st, a);
        return bg_rb<bf16_t, 8>(rb, jm, grid, lds, st, a);
    }
    if (sl <= 2) return bg_rb<float, 2>(rb, jm, grid, lds, st, a);
    return bg_rb<float, 4>(rb, jm, grid, lds, st, a);
}

}  // namespace bl
