// bmma.hip -- BitLinear for 1..64 quantized tokens on the int8 matrix cores.
//
// The product of a few dozen tokens with the packed weights ("穿越1比特的奇幻旅程",
// section 推理实现 / GPU端) reads every packed weight once from HBM, and every
// token's int8 row once per workgroup that needs it, from L2. A CU moves data
// at a rate set by how much it can keep in flight (about 67 GB/s from L2 and
// 26 GB/s from HBM per CU), so what decides the time is the bytes per
// workgroup, k * (16*TB tokens + 4 bytes * 16*RB rows): a workgroup owns a
// tile of RB 16-row blocks and TB 16-token blocks, and when the rows alone
// would leave few workgroups carrying many tokens the tokens are split over
// TS workgroups (TB = ceil(m / (16 TS))). The TS workgroups of one row tile
// get block ids 8 apart, so they land on the same XCD (workgroups go
// round-robin over the 8 XCDs) at about the same time and share its L2 copy
// of the tile's weights.
//  * The W waves split the chunk quads (4 x 64 inputs) of k into contiguous
//    ranges (W = 8..12, as many as make the busiest wave's share smallest:
//    10 waves of one quad for 2560 inputs rather than 8 waves of one or two),
//    and each wave works alone until the final reduction: it copies
//    the 16*TB token rows' bytes of its own quads into its own LDS region by
//    direct global->LDS loads (16 lanes per token and load: 256 contiguous
//    bytes, whole cache lines), then requests the packed weights of its quads
//    into registers (lane (h, r): the 16 bytes of chunk 4q+h of row r of each
//    row block), so that one wait for all but those weight loads covers its
//    rows. Token t's 16 pieces of a quad are stored rotated by t, so the
//    operand reads below, 16 tokens at one offset, fall on distinct banks.
//  * Step s of a quad: dword s of the weight bytes, expanded to 16 codes in
//    the qperm byte order, is operand A of v_mfma_i32_16x16x64_i8 against
//    operand B, the qperm bytes 16s..16s+15 of chunk 4q+h of token r (one
//    ds_read_b128). Chunks past k re-read the last chunk with their weight
//    word masked to code 0, which adds nothing.
//  * The waves' partial 16x16 blocks meet in LDS; the epilogue subtracts
//    sum_k q per token, applies the token's scale (one per token, computed
//    once) and stores y (or h of the gated FFN, or the bare int32 sums).
// Every sum is an exact integer, so the split over waves, workgroups and
// quads does not change any result.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kBmRegBudget = 64;  // VGPRs for the up-front weight words (NQ * NA * RB * 4)
constexpr int kBmLdsMax = 160 * 1024 - 1024;  // dynamic LDS (the rest: token scales and sums)

struct BmmaArgs {
    const int8_t *qp;  // qperm rows [>= m rounded up to 16 * TB][kp]
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
    int row_tiles;  // ceil(n / (16 RB))
    int ts;         // token slices
    int chunks;     // kp / 64
};

// LDS bytes of one wave: its quads' token rows, or later its partial sums
constexpr int bmma_wave_lds(int rb, int tb, int nq, int na)
{
    return nq * tb * 4096 > na * rb * tb * 1024 ? nq * tb * 4096 : na * rb * tb * 1024;
}
// the tiles that fit W waves: the up-front weight words within kBmRegBudget
// VGPRs, and with the accumulators within what W waves leave each (two waves
// per SIMD up to W = 8: 256 VGPRs; three: 168, less ~40 for addresses and
// operands); the waves' LDS within the CU's
constexpr bool bmma_fits(int rb, int tb, int nq, int na, int w)
{
    const int vgprs = w <= 8 ? 256 : 168;
    return nq * na * rb * 4 <= kBmRegBudget && nq * na * rb * 4 + na * rb * tb * 4 + 40 <= vgprs &&
           w * bmma_wave_lds(rb, tb, nq, na) <= kBmLdsMax;
}

template <int RB, int TB, int NQ, int EPI, int W>
__global__ __launch_bounds__(64 * W) void bmma_kernel(BmmaArgs a)
{
    constexpr int kBmW = W, kBmT = 64 * W;  // waves and threads per workgroup
    constexpr bool DUAL = EPI == EPI_GATE;
    constexpr int NA = DUAL ? 2 : 1;
    constexpr int WL = bmma_wave_lds(RB, TB, NQ, NA);
    constexpr int NW = NQ * NA * RB;  // weight loads per lane
    constexpr int RW = 16 * RB;       // rows of a tile
    extern __shared__ __align__(16) int8_t lds[];  // per wave: token rows, then partial sums
    __shared__ int tok_sq[16 * TB];
    __shared__ float tok_sc[NA][16 * TB];

    // block id -> (row tile, token slice): groups of 8 * TS ids, id % 8 the
    // row tile inside the group, (id / 8) % TS the token slice
    const int b = blockIdx.x;
    const int grp = b / (8 * a.ts), in = b - grp * 8 * a.ts;
    const int tile = grp * 8 + (in & 7), tsl = in >> 3;
    if (tile >= a.row_tiles) return;  // whole workgroup: the grid covers whole groups

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lh = lane >> 4;
    const int64_t r0 = (int64_t)tile * RW;
    const int rows = (int)(a.n - r0 < RW ? a.n - r0 : RW);
    const int64_t t0 = (int64_t)tsl * 16 * TB;
    const int toks = (int)(a.m - t0 < 16 * TB ? a.m - t0 : 16 * TB);
    const int C = a.chunks, NQT = (C + 3) >> 2;                    // chunks, quads of the row
    const int qb = wave * NQT / kBmW, qe = (wave + 1) * NQT / kBmW;  // this wave's quads [qb, qe)
    int8_t *wl = lds + wave * WL;                                  // this wave's LDS

    // 0. the tile's token code sums and scales, and gamma, requested first
    int my_sq = 0;
    float my_s = 0.0f, g0 = 0.0f, g1 = 0.0f;
    if (tid < toks) {
        my_sq = a.sumq[t0 + tid];
        if constexpr (EPI != EPI_ACC) {
            my_s = a.s[t0 + tid];
            g0 = a.gamma0[0];
            if constexpr (DUAL) g1 = a.gamma1[0];
        }
    }

    // 1. the token rows of this wave's quads into its LDS: load i of quad j
    //    covers tokens 4i..4i+3 (16 lanes each); slot p of token t holds its
    //    piece (p - t) mod 16 of the quad. Quads past the range, and loads
    //    whose four tokens are all past the tile's last token, are not issued
    //    (the products of those LDS slots belong to tokens that are dropped).
    {
        const uint32_t wl0 = lds_addr(wl);
        const int8_t *base = a.qp + t0 * a.kp;
        const int p = lane & 15;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            if (qb + j >= qe) break;  // uniform
            const int q = qb + j;
#pragma unroll
            for (int i = 0; i < 4 * TB; ++i) {
                if (4 * i >= toks) break;  // uniform: rows past the tile's tokens are not needed
                const int t = 4 * i + (lane >> 4);
                const int src = (p - t) & 15;
                // pieces past the row (the last quad of a row whose chunk
                // count is not a multiple of 4) re-read piece 0 of the quad:
                // their weight words are masked
                const int off = 256 * q + 16 * src < (int)a.kp ? 256 * q + 16 * src : 256 * q;
                dma16(base, (uint32_t)(t * (int)a.kp + off), wl0 + (uint32_t)((j * 16 * TB + 4 * i) * 256));
            }
        }
    }

    // 2. every weight word of this wave (after the rows, so that waiting for
    //    the rows does not wait for them): chunk 4q+h of row r of each row
    //    block; quads past the range re-read the wave's first (unused), chunks
    //    past k the last chunk (masked to code 0 at use)
    v4u wv[NQ][NA][RB];
    uint32_t wmask[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int q = qb + j < qe ? qb + j : (qb < NQT ? qb : NQT - 1);
        const int c = 4 * q + lh;
        wmask[j] = c < C ? 0xFFFFFFFFu : 0u;
        const int cc = c < C ? c : C - 1;
#pragma unroll
        for (int mat = 0; mat < NA; ++mat)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int r = 16 * rb + lr < rows ? 16 * rb + lr : rows - 1;  // extra rows re-read the last
                wv[j][mat][rb] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4u *>((mat ? a.w1 : a.w0) + (r0 + r) * a.ldw + cc * 16));
            }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm<NW, 15>());  // this wave's rows have landed
    asm volatile("" ::: "memory");

    // 3. products: per quad and step, the B operand of token 16 tb + r from LDS
    v4i acc[NA][RB][TB];
#pragma unroll
    for (int mat = 0; mat < NA; ++mat)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) acc[mat][rb][tb] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        if (qb + j >= qe) break;  // uniform
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v4i bq[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int t = 16 * tb + lr;
                bq[tb] = *reinterpret_cast<const v4i *>(wl + (j * 16 * TB + t) * 256 + ((4 * lh + s + t) & 15) * 16);
            }
#pragma unroll
            for (int mat = 0; mat < NA; ++mat)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const v4i av = expand_codes4(wv[j][mat][rb][s] & wmask[j]);
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb)
                        acc[mat][rb][tb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bq[tb], acc[mat][rb][tb], 0, 0, 0);
                }
        }
    }

    // 4. the partial blocks over the wave's own rows (its reads of them are
    //    earlier in its LDS queue); C[row][token]: lane (h, r) holds rows
    //    4h + v (v = 0..3) of token r of its block
    int *part = reinterpret_cast<int *>(wl);  // [NA][RB][TB][4][64]
#pragma unroll
    for (int mat = 0; mat < NA; ++mat)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int v = 0; v < 4; ++v) part[(((mat * RB + rb) * TB + tb) * 4 + v) * 64 + lane] = acc[mat][rb][tb][v];
    if (tid < toks) {
        tok_sq[tid] = my_sq;
        if constexpr (EPI != EPI_ACC) {
            tok_sc[0][tid] = token_scale(my_s, g0, a.qmax);
            if constexpr (DUAL) tok_sc[NA - 1][tid] = token_scale(my_s, g1, a.qmax);
        }
    }
    __syncthreads();

    // 5. epilogue: item i of a matrix's partial blocks, [RB][TB][v][lane]
    //    in the order every wave wrote them, so that consecutive threads read
    //    consecutive words of the eight waves' blocks (no bank conflicts);
    //    lane l of block (rb, tb), register v, is token 16 tb + l % 16 and row
    //    16 rb + 4 (l / 16) + v
    for (int i = tid; i < RB * TB * 256; i += kBmT) {
        const int l = i & 63, v = (i >> 6) & 3, rt = i >> 8;
        const int tb = rt % TB, rb = rt / TB;
        const int t = 16 * tb + (l & 15), row = 16 * rb + 4 * (l >> 4) + v;
        if (t >= toks || row >= rows) continue;
        const int sq = tok_sq[t];
        int va = -sq, vb = -sq;
#pragma unroll
        for (int w = 0; w < kBmW; ++w) {
            const int *pw = reinterpret_cast<const int *>(lds + w * WL);
            va += pw[i];
            if constexpr (DUAL) vb += pw[RB * TB * 256 + i];
        }
        const int64_t o = (t0 + t) * a.n + r0 + row;
        if constexpr (EPI == EPI_ACC) {
            a.acc_out[o] = va;
        } else if constexpr (DUAL) {
            a.out[o] = sq_relu_gate((float)va * tok_sc[0][t], (float)vb * tok_sc[NA - 1][t]);
        } else {
            a.out[o] = (float)va * tok_sc[0][t];
            if (a.acc_out) a.acc_out[o] = va;
        }
    }
}

// ---------------------------------------------------------------- host side

namespace {

struct BmmaShape {
    int rb = 0, tb = 0, ts = 0, nq = 0, w = 0;
};

// quads per wave with w waves: ceil(ceil(C / 4) / w). With 8 waves at most 4
// fit (8 waves x 4 quads x 16 tokens x 256 bytes of LDS), i.e. rows of up to
// 8192 inputs; longer ones go to the skinny kernel.
int64_t bmma_nq(int64_t C, int w = 8) { return ceil_div(ceil_div(C, (int64_t)4), (int64_t)w); }

// Waves per workgroup: the count among 8, 9, 10 and 12 that gives the busiest
// wave the fewest quads (the fewest waves among equals), as long as the
// smallest tile fits. The workgroup's bytes do not change with it; what does
// is how long its slowest wave runs: with 2560 inputs (10 quads) 8 waves
// leave two waves with two quads while the others wait for them at the final
// barrier. (16 waves of two quads for 6912 inputs measured slower than 9 of
// three: 25.7 against 25.5 us for a 2B layer at 8 tokens.)
int bmma_waves(int64_t C, int na)
{
    int best = 8;
    for (int w : {9, 10, 12})
        if (bmma_nq(C, w) < bmma_nq(C, best) && bmma_fits(1, 1, (int)bmma_nq(C, w), na, w)) best = w;
    return best;
}

// The tile for m tokens, n rows, kp inputs: among RB in {1, 2, 4} and TB in
// 1..4 (TS = ceil(m / 16 TB) token slices), the one whose busiest CU takes
// the least time: its token rows from L2 at about 67 GB/s and its weights
// from HBM at about 26 GB/s (what one CU keeps in flight over each latency),
// workgroups beyond the 256 CUs in further rounds, with the MFMA issue time
// (16 cycles per step, W / 4 waves per SIMD, 2.4 GHz) as the floor.
BmmaShape bmma_shape(int64_t m, int64_t n, int64_t kp, bool dual)
{
    const int na = dual ? 2 : 1;
    const int64_t C = kp / 64;
    const int w = bmma_waves(C, na);
    const int64_t nq = bmma_nq(C, w);
    BmmaShape best;
    double best_cost = 0.0;
    for (int rb = 1; rb <= 4; rb *= 2) {
        for (int tb = 1; tb <= 4; ++tb) {
            if (!bmma_fits(rb, tb, (int)nq, na, w)) continue;
            const int64_t ts = ceil_div(m, (int64_t)(16 * tb));
            const int64_t tiles = ceil_div(n, (int64_t)(16 * rb));
            const int64_t rounds = ceil_div(tiles * ts, (int64_t)256);
            const double mem_ns = 16.0 * tb * kp / 67.0 + 4.0 * rb * na * kp / 26.0;
            const double mfma_ns = (double)nq * 4 * na * rb * tb * 16.0 * (w / 4.0) / 2.4;
            const double cost = (double)rounds * (mem_ns > mfma_ns ? mem_ns : mfma_ns);
            if (best.rb == 0 || cost < best_cost) {
                best_cost = cost;
                best.rb = rb; best.tb = tb; best.ts = (int)ts; best.nq = (int)nq; best.w = w;
            }
        }
    }
    return best;
}

template <int RB, int TB, int NQ, int EPI, int W>
hipError_t bm_launch(const BmmaArgs &a, dim3 grid, hipStream_t st)
{
    constexpr int NA = EPI == EPI_GATE ? 2 : 1;
    if constexpr (bmma_fits(RB, TB, NQ, NA, W)) {
        const int lds = W * bmma_wave_lds(RB, TB, NQ, NA);
        const auto kern = bmma_kernel<RB, TB, NQ, EPI, W>;
        static LdsLimit lim;
        if (hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kern), (int)lds, lim)) return e;
        hipLaunchKernelGGL(kern, grid, dim3(64 * W), (size_t)lds, st, a);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <int RB, int TB, int NQ, int W>
hipError_t bm_epi(const BmmaArgs &a, int epi, dim3 grid, hipStream_t st)
{
    switch (epi) {
    case EPI_Y: return bm_launch<RB, TB, NQ, EPI_Y, W>(a, grid, st);
    case EPI_ACC: return bm_launch<RB, TB, NQ, EPI_ACC, W>(a, grid, st);
    default: return bm_launch<RB, TB, NQ, EPI_GATE, W>(a, grid, st);
    }
}

// quads per wave: at most ceil(32 / W) (rows of up to 8192 inputs)
template <int RB, int TB, int W>
hipError_t bm_nq(int nq, const BmmaArgs &a, int epi, dim3 grid, hipStream_t st)
{
    switch (nq) {
    case 1: return bm_epi<RB, TB, 1, W>(a, epi, grid, st);
    case 2: return bm_epi<RB, TB, 2, W>(a, epi, grid, st);
    case 3: return bm_epi<RB, TB, 3, W>(a, epi, grid, st);
    case 4:
        if constexpr (W <= 10) return bm_epi<RB, TB, 4, W>(a, epi, grid, st);
        else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int RB, int W>
hipError_t bm_tb(int tb, int nq, const BmmaArgs &a, int epi, dim3 grid, hipStream_t st)
{
    switch (tb) {
    case 1: return bm_nq<RB, 1, W>(nq, a, epi, grid, st);
    case 2: return bm_nq<RB, 2, W>(nq, a, epi, grid, st);
    case 3: return bm_nq<RB, 3, W>(nq, a, epi, grid, st);
    case 4: return bm_nq<RB, 4, W>(nq, a, epi, grid, st);
    default: return hipErrorInvalidValue;
    }
}

template <int W>
hipError_t bm_rb(const BmmaShape &sh, const BmmaArgs &a, int epi, dim3 grid, hipStream_t st)
{
    switch (sh.rb) {
    case 1: return bm_tb<1, W>(sh.tb, sh.nq, a, epi, grid, st);
    case 2: return bm_tb<2, W>(sh.tb, sh.nq, a, epi, grid, st);
    default: return bm_tb<4, W>(sh.tb, sh.nq, a, epi, grid, st);
    }
}

}  // namespace

bool bmma_supported(int64_t m, int64_t kp, bool dual)
{
    if (m < 1 || m > 64 || kp < 64) return false;
    const int64_t nq = bmma_nq(kp / 64);
    return nq <= 4 && bmma_fits(1, 1, (int)nq, dual ? 2 : 1, 8);
}

hipError_t launch_bmma(const GemmProblem &p, hipStream_t st)
{
    const bool dual = p.epi == EPI_GATE;
    BmmaArgs a;
    a.qp = p.qp; a.kp = p.kp; a.s = p.s; a.sumq = p.sumq; a.m = p.m; a.n = p.n;
    a.w0 = p.w0; a.w1 = dual ? p.w1 : p.w0; a.ldw = p.ldw;
    a.gamma0 = p.gamma0; a.gamma1 = dual ? p.gamma1 : p.gamma0;
    a.out = p.out; a.acc_out = p.acc_out; a.qmax = p.qmax;
    a.chunks = (int)(p.kp / 64);
    const BmmaShape sh = bmma_shape(p.m, p.n, p.kp, dual);
    if (sh.rb == 0) return hipErrorInvalidValue;
    a.ts = sh.ts;
    a.row_tiles = (int)ceil_div(p.n, (int64_t)(16 * sh.rb));
    const dim3 grid((unsigned)(ceil_div((int64_t)a.row_tiles, (int64_t)8) * 8 * sh.ts));
    switch (sh.w) {
    case 8: return bm_rb<8>(sh, a, p.epi, grid, st);
    case 9: return bm_rb<9>(sh, a, p.epi, grid, st);
    case 10: return bm_rb<10>(sh, a, p.epi, grid, st);
    default: return bm_rb<12>(sh, a, p.epi, grid, st);
    }
}

}  // namespace bl
