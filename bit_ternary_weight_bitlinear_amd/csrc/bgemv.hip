// bgemv.hip -- BitLinear for 5..64 tokens (batched decode) on gfx950.
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
//    the 16 qperm bytes of token r (of each 16-token block: passes of 32
//    tokens run two MFMAs per operand) at the same inputs, read from LDS;
//  * for m*k up to 32768 the m tokens are quantized once per workgroup, from
//    raw words loaded before the weights and converted after the weight loads
//    are issued: a per-token absmax (16-lane DPP maxima over the at most two
//    tokens a wave's 64 groups touch, merged by LDS atomics), one division per
//    token, then codes into LDS in qperm order (rows of whole chunk quads,
//    zero past k, plus 16 bytes: the 16 rows of one read phase fall on
//    different banks) and sum_k q per token.
//    Larger m*k would cost every workgroup too much arithmetic (2 us of VALU
//    per CU at 8 x 6912 inputs); there, and above 16 tokens, the quantization
//    kernel runs first and this one copies its int8 rows, scales and sums into
//    LDS instead (PREQ), in passes of 32 tokens (when 32 rows fit the LDS) or
//    16, while the weights stay in registers;
//  * the waves' partial 16x16 blocks meet in LDS; the epilogue subtracts
//    sum_k q, rescales, stores y (and the int32 sums if asked).
// Integer sums are exact, so the split over waves and the order of the adds
// do not change results.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kBT = 512;       // threads per workgroup (8 waves)
constexpr int kBW = kBT / 64;  // waves per workgroup
constexpr int kBMaxTok = 32;   // tokens per pass: two 16-token MFMA blocks (the second: pre-quantized rows only)
constexpr int kBMaxTokens = 64;  // tokens per launch (passes of 16 or 32)
constexpr int kBMaxRows = 32;  // at most two 16-row blocks per workgroup
constexpr int kBMaxK = 8192;

struct BgemvArgs {
    const void *x;  // bf16 / fp32 activations, or (PREQ) qperm int8 rows of kp bytes
    const float *pre_s;
    const int32_t *pre_sumq;
    int64_t m, k, kp, n;
    const uint8_t *w;
    int64_t ldw;
    const float *gamma;
    float *out;
    int32_t *acc_out;
    float qmax;
    int rows_per_wg;  // R
    int chunks;       // kp / 64
};

// RB: 16-row blocks per workgroup (1 or 2). JM: quads per wave. SL: activation
// groups of 16 inputs per thread (covering all m * k / 16 of them), or with
// PREQ 16-byte words of the quantized rows (all m * kp / 16 of them).
template <typename T, int RB, int JM, int SL, bool PREQ, int MB>
__global__ __launch_bounds__(kBT) void bgemv_kernel(BgemvArgs a)
{
    static_assert(PREQ || MB == 1, "the fused quantization handles one token block");
    extern __shared__ __align__(16) int8_t lds[];  // token rows [TP][QS], then partial sums [kBW][MB][4][64]
    __shared__ unsigned tok_max[kBMaxTok];
    __shared__ int tok_sum[kBMaxTok];
    __shared__ float tok_inv[kBMaxTok], tok_s[kBMaxTok];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lh = lane >> 4;
    const int M = (int)a.m;
    // tokens go through LDS in passes of TP (one pass unless PREQ); the weights
    // stay in registers across the passes
    constexpr int TP = 16 * MB;
    const int P = PREQ ? (M + TP - 1) / TP : 1;
    const int R = a.rows_per_wg, C = a.chunks;
    // LDS token rows: TP of them, each 16 * GQ bytes of qperm codes (whole
    // quads of chunks; codes past kp and rows past the pass's tokens are zero,
    // so the products read their operands without selects) plus 16 bytes, so
    // the 16 rows of one read phase fall on different banks
    const int nq = (C + 3) >> 2;
    const int GQ = 16 * nq;
    const int QS = 16 * GQ + 16;
    int8_t *q_lds = lds;
    int *part = reinterpret_cast<int *>(lds + TP * QS);
    const int64_t r0 = (int64_t)blockIdx.x * R;
    const int rows = (int)((a.n - r0) < R ? (a.n - r0) : R);
    const T *x = static_cast<const T *>(a.x);
    const int GP = (int)(a.kp / 16);
    const int G = PREQ ? GP : (int)(a.k / 16);  // fused: k % 16 == 0

    if (tid < kBMaxTok) {
        tok_max[tid] = 0u;
        tok_sum[tid] = 0;
    }

    // 1. activation loads of a pass (raw words; with PREQ the quantized rows'
    //    16-byte words); slots no thread needs are not loaded (uniform). Slot s
    //    of a thread is the pass's flat group f = tid + s * kBT, i.e. group
    //    f % G of token f / G; a token row is exactly G groups wide (k = 16 G,
    //    or with PREQ rows of kp = 16 G bytes), so its address is 16 f past
    //    the pass's first row and the division waits until the loads are out
    constexpr int XQ = PREQ ? 1 : (int)sizeof(T);  // 16-byte words per group
    uint4 xq[SL][XQ];
    int slot_f[SL], slot_t[SL], slot_g[SL];
    auto load_pass = [&](int t0, int mp) {
        const int ng = mp * G;
        const int64_t g0 = (int64_t)t0 * G;  // the pass's first group
#pragma unroll
        for (int s = 0; s < SL; ++s) {
            slot_f[s] = min(tid + s * kBT, ng - 1);
            if (s * kBT < ng) {
                const int64_t e = 16 * (g0 + slot_f[s]);  // elements (PREQ: bytes)
                const uint4 *p = PREQ ? reinterpret_cast<const uint4 *>(static_cast<const int8_t *>(a.x) + e)
                                      : reinterpret_cast<const uint4 *>(x + e);
#pragma unroll
                for (int q = 0; q < XQ; ++q) xq[s][q] = p[q];
            } else {
#pragma unroll
                for (int q = 0; q < XQ; ++q) xq[s][q] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto split_slots = [&] {
#pragma unroll
        for (int s = 0; s < SL; ++s) {
            slot_t[s] = slot_f[s] / G;
            slot_g[s] = slot_f[s] - slot_t[s] * G;
        }
    };
    const int Mp0 = min(M, TP);
    load_pass(0, Mp0);  // the first pass's before the weights
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
    split_slots();

    // zero codes: each row's groups G .. GQ, and the rows past the first
    // pass's tokens
    for (int i = tid; i < Mp0 * (GQ - G); i += kBT) {
        const int t = i / (GQ - G), g = G + (i - t * (GQ - G));
        *reinterpret_cast<uint4 *>(q_lds + t * QS + g * 16) = make_uint4(0, 0, 0, 0);
    }
    for (int i = tid; i < (TP - Mp0) * GQ; i += kBT) {
        const int t = Mp0 + i / GQ, g = i - (t - Mp0) * GQ;
        *reinterpret_cast<uint4 *>(q_lds + t * QS + g * 16) = make_uint4(0, 0, 0, 0);
    }
    // PREQ: a pass's quantized rows into LDS, with their scales and sums
    auto store_pass = [&](int t0, int mp) {
        if (tid < mp) {
            tok_s[tid] = a.pre_s[t0 + tid];
            tok_sum[tid] = a.pre_sumq[t0 + tid];
        }
        const int ng = mp * G;
#pragma unroll
        for (int s = 0; s < SL; ++s)
            if (tid + s * kBT < ng)
                *reinterpret_cast<uint4 *>(q_lds + slot_t[s] * QS + slot_g[s] * 16) = xq[s][0];
    };
    if constexpr (PREQ) {
        // the first pass outside the loop: it waits for its rows only, not
        // for the weights requested after them
        store_pass(0, Mp0);
        __syncthreads();
    }

    for (int pass = 0; pass < P; ++pass) {
    const int t0 = pass * TP, Mp = min(TP, M - t0), NG = Mp * G;
    if constexpr (PREQ) {
        if (pass > 0) {
            load_pass(t0, Mp);
            split_slots();
            store_pass(t0, Mp);
            // a short last pass: its rows past the tokens read as zero
            for (int i = tid; i < (TP - Mp) * G; i += kBT) {
                const int t = Mp + i / G, g = i - (t - Mp) * G;
                *reinterpret_cast<uint4 *>(q_lds + t * QS + g * 16) = make_uint4(0, 0, 0, 0);
            }
            __syncthreads();
        }
    } else {
    // 3. per-token absmax. The 64 groups of one wave and slot belong to at most
    //    two tokens (t0 and t0 + 1: a token has G >= 64 groups); each 16-lane
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
        const int u0 = f0 / G;
        const float m0 = row16_max(valid && slot_t[s] == u0 ? mx : 0.0f);
        const float m1 = row16_max(valid && slot_t[s] != u0 ? mx : 0.0f);
        if (lr == 0) {
            atomicMax(&tok_max[u0], __float_as_uint(m0));
            if (u0 + 1 < Mp) atomicMax(&tok_max[u0 + 1], __float_as_uint(m1));
        }
    }
    __syncthreads();
    if (tid < Mp) {
        const float st = fmaxf(__uint_as_float(tok_max[tid]), kEps);
        tok_s[tid] = st;
        tok_inv[tid] = 127.0f / st;
    }
    __syncthreads();

    // 4. codes into LDS (qperm order) and sum_k q per token (inputs past k
    //    were zeroed above)
#pragma unroll
    for (int s = 0; s < SL; ++s) {
        const int f0 = wave * 64 + s * kBT;
        if (f0 >= NG) continue;
        const bool valid = tid + s * kBT < NG;
        int sum = 0;
        if (valid) {
            uint4 pv;
            sum = quant_group(xk[s], tok_inv[slot_t[s]], &pv, nullptr);
            *reinterpret_cast<uint4 *>(q_lds + slot_t[s] * QS + slot_g[s] * 16) = pv;
        }
        const int u0 = f0 / G;
        const int s0 = row16_sum(valid && slot_t[s] == u0 ? sum : 0);
        const int s1 = row16_sum(valid && slot_t[s] != u0 ? sum : 0);
        if (lr == 0) {
            atomicAdd(&tok_sum[u0], s0);
            if (u0 + 1 < Mp) atomicAdd(&tok_sum[u0 + 1], s1);
        }
    }
    __syncthreads();
    }

    // 5. products: per quad, four MFMAs (dword s of each lane's 16 packed bytes
    //    against the qperm bytes of token lr at the same inputs); tokens past
    //    the pass and chunks past the row read zero codes (with two token
    //    blocks each expanded operand feeds two MFMAs)
    v4i acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        const int cq = wave / RB + (kBW / RB) * j;
        if (cq < nq) {  // uniform
            const int8_t *qc = q_lds + lr * QS + (4 * cq + lh) * 64;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const v4i av = expand_codes4(wv[j][s]);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        av, *reinterpret_cast<const v4i *>(qc + 16 * mb * QS + s * 16), acc[mb], 0, 0, 0);
            }
        }
    }
    // C[row][token]: lane (h, r) holds rows 4h + v (v = 0..3) of token 16*mb + r
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[((wave * MB + mb) * 4 + v) * 64 + lane] = acc[mb][v];
    __syncthreads();

    // 6. epilogue: item -> (row block, token block, register v, lane), summed
    //    over the waves of its row block
    for (int e = tid; e < RB * MB * 256; e += kBT) {
        const int eb = e / (MB * 256), rem = e - eb * (MB * 256);
        const int mb = rem >> 8, v = (rem >> 6) & 3, el = rem & 63;
        const int row = 16 * eb + 4 * (el >> 4) + v, t = 16 * mb + (el & 15);
        if (row < rows && t < Mp) {
            int va = -tok_sum[t];
#pragma unroll
            for (int w = eb; w < kBW; w += RB) va += part[((w * MB + mb) * 4 + v) * 64 + el];
            const int64_t o = (int64_t)(t0 + t) * a.n + r0 + row;
            a.out[o] = (float)va * token_scale(tok_s[t], a.gamma[0], a.qmax);
            if (a.acc_out) a.acc_out[o] = va;
        }
    }
    if (pass + 1 < P) __syncthreads();  // LDS rows, sums and scales are rewritten next pass
    }
}

// ---------------------------------------------------------------- host side

static int bgemv_slots(int64_t words) { return (int)ceil_div(words, (int64_t)kBT); }

constexpr size_t kBLdsMax = 150 * 1024;
// token blocks per pass: two when 32 token rows fit the LDS
// LDS bytes: 16 * mb token rows of whole chunk quads plus 16 bytes, then the
// waves' partial sums
static size_t bgemv_lds(int64_t kp, int mb)
{
    return (size_t)16 * mb * (round_up(kp, 256) + 16) + (size_t)kBW * mb * 4 * 64 * 4;
}
static int bgemv_mb(int64_t m, int64_t kp)
{
    return m > 16 && bgemv_lds(kp, 2) <= kBLdsMax ? 2 : 1;
}

int bgemv_mode(int64_t m, int64_t k, bool bf16)
{
    if (m < 5 || m > kBMaxTokens || k > kBMaxK) return 0;
    // fused: one token block, whole 16-input groups, at least 64 of them per
    // token (a wave's groups touch two tokens at most) and few enough inputs
    // that every workgroup may quantize them all
    if (m <= 16 && k % 16 == 0 && k >= 1024 && m * k <= 32768 && bgemv_slots(m * k / 16) <= (bf16 ? 8 : 4))
        return 1;
    return bgemv_prequant_supported(m, k) ? 2 : 0;
}

bool bgemv_prequant_supported(int64_t m, int64_t k)
{
    if (m < 5 || m > kBMaxTokens || k > kBMaxK) return false;
    const int64_t kp = round_up(k, 64);
    const int mb = bgemv_mb(m, kp);
    return bgemv_slots(16 * mb * kp / 16) <= 16 && bgemv_lds(kp, mb) <= kBLdsMax;
}

namespace {

template <typename T, int RB, int JM, int SL, bool PREQ, int MB>
hipError_t bg_launch(dim3 grid, size_t lds, hipStream_t st, const BgemvArgs &a)
{
    auto kern = bgemv_kernel<T, RB, JM, SL, PREQ, MB>;
    static LdsLimit lim;
    if (hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kern), (int)lds, lim)) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kBT), lds, st, a);
    return hipGetLastError();
}

template <typename T, int RB, int SL, bool PREQ, int MB>
hipError_t bg_jm(int jm, dim3 grid, size_t lds, hipStream_t st, const BgemvArgs &a)
{
    if (jm <= 1) return bg_launch<T, RB, 1, SL, PREQ, MB>(grid, lds, st, a);
    if (jm <= 2) return bg_launch<T, RB, 2, SL, PREQ, MB>(grid, lds, st, a);
    if (jm <= 3) return bg_launch<T, RB, 3, SL, PREQ, MB>(grid, lds, st, a);
    if (jm <= 4) return bg_launch<T, RB, 4, SL, PREQ, MB>(grid, lds, st, a);
    if (jm <= 6) return bg_launch<T, RB, 6, SL, PREQ, MB>(grid, lds, st, a);
    return bg_launch<T, RB, 8, SL, PREQ, MB>(grid, lds, st, a);
}

template <typename T, int SL, bool PREQ, int MB = 1>
hipError_t bg_rb(int rb, int jm, dim3 grid, size_t lds, hipStream_t st, const BgemvArgs &a)
{
    return rb == 1 ? bg_jm<T, 1, SL, PREQ, MB>(jm, grid, lds, st, a) : bg_jm<T, 2, SL, PREQ, MB>(jm, grid, lds, st, a);
}

template <int SL>
hipError_t bg_preq(int mb, int rb, int jm, dim3 grid, size_t lds, hipStream_t st, const BgemvArgs &a)
{
    return mb == 1 ? bg_rb<int8_t, SL, true, 1>(rb, jm, grid, lds, st, a) : bg_rb<int8_t, SL, true, 2>(rb, jm, grid, lds, st, a);
}

}  // namespace

hipError_t launch_bgemv(const GemvProblem &p, hipStream_t st)
{
    BgemvArgs a;
    const bool preq = p.pre_s != nullptr;
    a.x = p.x; a.pre_s = p.pre_s; a.pre_sumq = p.pre_sumq;
    a.m = p.m; a.k = p.k; a.kp = p.kp; a.n = p.n;
    a.w = p.w0; a.ldw = p.ldw; a.gamma = p.gamma0;
    a.out = p.out; a.acc_out = p.acc_out; a.qmax = p.qmax;
    a.chunks = (int)(p.kp / 64);
    int64_t r = ceil_div(p.n, (int64_t)256);
    if (r > kBMaxRows) r = kBMaxRows;
    a.rows_per_wg = (int)r;
    const int rb = r > 16 ? 2 : 1;
    const int64_t nq = ceil_div((int64_t)a.chunks, (int64_t)4);
    const int jm = (int)ceil_div(nq, (int64_t)(kBW / rb));  // <= 8: kp <= 8192
    const dim3 grid((unsigned)ceil_div(p.n, r));
    if (preq) {
        const int mb = bgemv_mb(p.m, p.kp);
        const size_t lds = bgemv_lds(p.kp, mb);
        const int sl = bgemv_slots((p.m < 16 * mb ? p.m : 16 * mb) * p.kp / 16);
        if (sl <= 2) return bg_preq<2>(mb, rb, jm, grid, lds, st, a);
        if (sl <= 4) return bg_preq<4>(mb, rb, jm, grid, lds, st, a);
        if (sl <= 8) return bg_preq<8>(mb, rb, jm, grid, lds, st, a);
        return bg_preq<16>(mb, rb, jm, grid, lds, st, a);
    }
    const size_t lds = bgemv_lds(p.kp, 1);
    const int sl = bgemv_slots(p.m * p.k / 16);
    if (p.bf16) {
        if (sl <= 2) return bg_rb<bf16_t, 2, false>(rb, jm, grid, lds, st, a);
        if (sl <= 4) return bg_rb<bf16_t, 4, false>(rb, jm, grid, lds, st, a);
        return bg_rb<bf16_t, 8, false>(rb, jm, grid, lds, st, a);
    }
    if (sl <= 2) return bg_rb<float, 2, false>(rb, jm, grid, lds, st, a);
    return bg_rb<float, 4, false>(rb, jm, grid, lds, st, a);
}

}  // namespace bl
