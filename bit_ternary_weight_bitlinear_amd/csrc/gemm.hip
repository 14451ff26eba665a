// gemm.hip -- BitLinear at m > 64 tokens on the gfx950 int8 matrix cores.
//
// At many tokens the W1.58A8 product ("穿越1比特的奇幻旅程", section 推理实现 / GPU端)
// is a dense contraction, so it runs on v_mfma_i32_32x32x32_i8 with the
// activations as operand A and the ternary codes as operand B:
//  * a workgroup owns a tile of 128*FM tokens x 32*FN output features. With
//    four waves, wave w takes tokens [32*FM*w, 32*FM*(w+1)) of it against all
//    32*FN features (FM*FN accumulator blocks of 32x32). 256-token tiles run
//    eight waves, two per SIMD: waves w and w+4 take the same tokens, one the
//    first (FN+1)/2 feature fragments and the other the rest, so while one
//    waits at a barrier or for LDS the other keeps the SIMD's matrix core busy
//    (same MFMA work per SIMD, half the accumulators per wave); 256x224
//    tiles run sixteen waves, four per SIMD, in four fragment groups;
//  * two LDS rings, filled by direct global->LDS loads (global_load_lds_dwordx4)
//    issued DB k-steps ahead: the qperm activation tile of each 64-input step
//    (64-byte rows) and the packed weight rows of that step (16-byte rows).
//    The loads take a scalar base (advanced by one step with scalar adds) and
//    a constant per-lane offset, and ring positions are scalar offsets, so the
//    loop spends its vector instructions on the weight expansion alone;
//  * the weights stay packed in LDS. Each lane reads the 8 packed bytes its
//    operand needs for a whole step (one ds_read_b64) and expands them in
//    registers: (w >> 2i) & 0x03030303 holds the codes of inputs 16g+4b+i,
//    exactly the qperm byte order of the activations. Lanes 0-31 take 16-input
//    groups {0,1} of the step, lanes 32-63 groups {2,3}: half-step h uses
//    group h + 2*(lane/32) on both operands;
//  * software pipelined by half steps: while one half's MFMAs run, the wave
//    reads the other half's activation fragments and the next step's packed
//    weights; one barrier per step, which waits only for the direct loads the
//    next step reads (the younger ones stay in flight across it). Two steps per
//    loop iteration let the packed-weight registers alternate without copies;
//  * the tile's per-token sum_k q and s arrive in LDS by direct loads in the
//    prologue and are read back four tokens at a time by the epilogue;
//  * activation rows are 64 bytes (four 16-byte slots), slot index XORed by
//    (row >> 2) & 3, so the sixteen lanes of each ds_read_b128 phase, reading
//    sixteen consecutive rows at one slot, cover all 64 banks once;
//  * tiles are ordered per XCD: workgroup i runs on XCD i % 8, so XCD x gets a
//    contiguous range of tiles that share their activation rows (L2 reuse);
//  * accumulator block layout: lane l holds feature n = l % 32 and tokens
//    m = 8*(v/4) + 4*(l/32) + v%4 in register v, so each store instruction
//    writes two 128-byte row segments;
//  * codes are w+1 in {0,1,2}; the epilogue subtracts sum_k q per token.
// Integer accumulation is exact; the fp32 rescale is the same operation
// sequence as on the decode path.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

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
    int64_t ldo;  // row stride of out / acc_out (>= n: a column range of a wider output)
    float qmax;
    int n_tiles, m_tiles;
};

// byte offset of (row, 16-byte group g) in a 64-byte-row LDS tile
__device__ inline int tile_off(int row, int g) { return row * 64 + ((g ^ ((row >> 2) & 3)) << 4); }

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// one v_lshrrev_b64 (written out: the compiler would split a 64-bit shift whose
// high bits are masked off into two 32-bit shifts)
template <int S>
__device__ inline uint64_t shr64(uint64_t v)
{
    uint64_t r;
    asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "i"(S), "v"(v));
    return r;
}

// Epilogue of one wave (y goes out with non-temporal stores; h of a gate/up
// pair with plain ones, since the requantization reads it right after and
// finds part of it in the caches: 22.3 against 26.5 us at 2048 x 14336):
// y = (float)(acc - sumq) * ((s / 127) * gamma) for its 32*FM tokens (tile
// rows tokw*32*FM ..) x its FN fragments of 32 features, starting at tile
// column 32*FOFF. tok_sq / tok_s hold sum_k q and s of the tile's tokens
// (LDS). Interior tiles store without bounds checks, one row pointer per token
// and immediate offsets per block.
template <int FM, int FN, int FOFF, int EPI>
__device__ __forceinline__ void store_tile(const GemmArgs &a, const v16i (&acc)[EPI == EPI_GATE ? 2 : 1][FM][FN],
                                           const int *tok_sq, const float *tok_s, int64_t m0, int64_t n0t,
                                           int tokw, int lrow, int lhalf)
{
    constexpr bool DUAL = EPI == EPI_GATE;
    constexpr int NA = DUAL ? 2 : 1;
    constexpr int BM = 128 * FM, BN = 32 * FN, WM = 32 * FM;
    const int64_t n0 = n0t + 32 * FOFF;
    float *const out = a.out;
    int32_t *const acc_out = a.acc_out;
    const int64_t M = a.m, N = a.n, LDO = a.ldo;
    float g0 = 0.0f, g1 = 0.0f;
    if constexpr (EPI != EPI_ACC) {
        g0 = a.gamma0[0];
        if constexpr (DUAL) g1 = a.gamma1[0];
    }
    auto epilogue = [&](auto full_c, auto acc_c) {
        constexpr bool FULL = decltype(full_c)::value;
        constexpr bool ACC = decltype(acc_c)::value;  // int32 results stored (as well)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = tokw * WM + fm * 32 + 8 * j + 4 * lhalf;  // tile row of register 4j
                const v4i sq = *reinterpret_cast<const v4i *>(tok_sq + r);
                float c0e[4] = {0.0f, 0.0f, 0.0f, 0.0f}, c1e[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (EPI != EPI_ACC) {
                    const float4 sv = *reinterpret_cast<const float4 *>(tok_s + r);
                    const float se[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        c0e[e] = token_scale(se[e], g0, a.qmax);
                        if constexpr (DUAL) c1e[e] = token_scale(se[e], g1, a.qmax);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t m = m0 + r + e;
                    if (!FULL && m >= M) continue;
                    const int64_t row = m * LDO + n0 + lrow;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        if (!FULL && n0 + fn * 32 + lrow >= N) continue;
                        const int va = acc[0][fm][fn][4 * j + e] - sq[e];
                        if constexpr (EPI != EPI_ACC) {
                            float o;
                            if constexpr (DUAL) o = sq_relu_gate((float)va * c0e[e], (float)(acc[NA - 1][fm][fn][4 * j + e] - sq[e]) * c1e[e]);
                            else o = (float)va * c0e[e];
                            if constexpr (DUAL) out[row + fn * 32] = o;
                            else __builtin_nontemporal_store(o, &out[row + fn * 32]);
                        }
                        if constexpr (ACC) __builtin_nontemporal_store(va, &acc_out[row + fn * 32]);
                    }
                }
            }
    };
    using T = std::true_type;
    using F = std::false_type;
    const bool full = m0 + BM <= M && n0 + BN <= N;
    if constexpr (EPI == EPI_ACC) {
        if (full) epilogue(T(), T());
        else epilogue(F(), T());
    } else if constexpr (EPI == EPI_Y) {
        if (acc_out) {
            if (full) epilogue(T(), T());
            else epilogue(F(), T());
        } else {
            if (full) epilogue(T(), F());
            else epilogue(F(), F());
        }
    } else {
        if (full) epilogue(T(), F());
        else epilogue(F(), F());
    }
}

// The work of one wave of a tile of 128*FM tokens x 32*FN features, run by NW
// waves: wave w takes tokens [32*FM*(w%4), 32*FM*(w%4+1)) of the tile against
// its FW fragments of 32 features starting at fragment FOFF. With NW = 4 every
// wave has all FN fragments; with NW = 8 (two waves per SIMD) waves 0-3 take
// the first (FN+1)/2 fragments and waves 4-7 the rest, so each SIMD keeps the
// same MFMA work with half the accumulators per wave, and one wave's barrier
// and LDS waits can be covered by the other's MFMAs; NW = 16 (four waves per
// SIMD) splits the fragments into four groups the same way. The direct loads
// of a step are spread over all NW waves (the packed weight rows over waves
// 0-3: WLOAD). SPB: 64-input steps per ring stage (1 or 2). With 2, the direct
// loads of a stage go out once per pair of steps and the barrier runs once per
// pair; the step count must be even. DB: stages requested ahead.
template <int FM, int FN, int EPI, int DB, int SPB, int NW, int FW, int FOFF, bool WLOAD>
__device__ __forceinline__ void gemm_waves(const GemmArgs &a, int8_t *smem, int wave, int64_t m0, int64_t n0)
{
    constexpr bool DUAL = EPI == EPI_GATE;
    constexpr int NA = DUAL ? 2 : 1;
    constexpr int BM = 128 * FM, BN = 32 * FN, WM = 32 * FM;
    static_assert(FM * FW * NA <= 16, "accumulators fit the 256 AGPRs");
    static_assert(NW == 4 || (NW == 8 && FM * FW * NA <= 8) || (NW == 16 && FM * FW * NA <= 4),
                  "two or four waves per SIMD: a half or a quarter of the accumulators");
    static_assert(FW >= 1, "every wave owns at least one fragment");
    static_assert(BN <= 256, "packed rows: one 64-row direct load per wave");
    static_assert(DB >= 3, "at least one stage of slack for the direct loads");
    static_assert(SPB == 1 || SPB == 2, "one or two steps per stage");
    constexpr int X_TILE = BM * 64;        // activation bytes per step
    constexpr int W_PK = 256 * 16;         // packed bytes per step and matrix (256 rows)
    constexpr int W_STAGE = NA * W_PK;     // packed bytes per step
    constexpr int XS = SPB * X_TILE, WS = SPB * W_STAGE;  // bytes per ring stage
    // Live stages: activations of stages S .. S+DB; packed weights of S+1 .. S+DB,
    // and with two steps per stage also S (its second step's weights are read
    // during its first step).
    constexpr int SBX = DB + 1;
    constexpr int SBW = SPB == 1 ? DB : DB + 1;
    constexpr int X_INSTR = BM / (16 * NW);  // activation direct loads per thread per step
    static_assert(X_INSTR * 16 * NW == BM, "activation rows split evenly over the waves");
    constexpr int DPS = SPB * (X_INSTR + (WLOAD ? NA : 0));  // direct loads per thread per stage
    constexpr int VM_SLACK = (DB - 2) * DPS;
    static_assert(VM_SLACK < 64, "vmcnt field");
    // LDS: xring[SBX][XS], wring[SBW][WS], then sum_k q and s of the tile's tokens
    constexpr int XR = 0, WR = SBX * XS, TQ = WR + SBW * WS, TS = TQ + BM * 4;
    const uint32_t lds0 = lds_addr(smem);

    const int lane = threadIdx.x & 63;
    const int tokw = wave & 3;  // token group of the tile
    const int lrow = lane & 31, lhalf = lane >> 5;

    const int nks = (int)(a.kp / 64);
    // direct-load sources: scalar bases advanced per step, constant per-lane offsets
    const int8_t *xbase = a.qp + m0 * a.kp;
    uint32_t xoff[X_INSTR];
#pragma unroll
    for (int i = 0; i < X_INSTR; ++i) {
        const int row = (i * NW + wave) * 16 + (lane >> 2);
        const int g = (lane & 3) ^ ((row >> 2) & 3);
        xoff[i] = (uint32_t)(row * a.kp + g * 16);
    }
    const uint8_t *wbase[NA];
#pragma unroll
    for (int mat = 0; mat < NA; ++mat) wbase[mat] = (mat == 0 ? a.w0 : a.w1) + n0 * a.ldw;
    uint32_t woff;
    {
        // rows past the tile or the matrix re-read a valid row (results dropped)
        int64_t n = n0 + min(wave * 64 + lane, BN - 1);
        n = n < a.n ? n : a.n - 1;
        woff = (uint32_t)((n - n0) * a.ldw);
    }
    // requests stage j (steps SPB*j ..) into the ring stages at byte offsets xo / wo
    auto dma_stage = [&](int j, uint32_t xo, uint32_t wo) {
#pragma unroll
        for (int sub = 0; sub < SPB; ++sub) {
            const int64_t ks = (int64_t)SPB * j + sub;
#pragma unroll
            for (int i = 0; i < X_INSTR; ++i)
                dma16(xbase + ks * 64, xoff[i], lds0 + XR + xo + sub * X_TILE + (i * NW + wave) * 1024);
            if constexpr (WLOAD) {
#pragma unroll
                for (int mat = 0; mat < NA; ++mat)
                    dma16(wbase[mat] + ks * 16, woff, lds0 + WR + wo + sub * W_STAGE + mat * W_PK + wave * 1024);
            }
        }
    };

    // LDS read addresses: per-lane bases, stage offsets added per step
    const uint32_t xl0 = XR + tile_off(tokw * WM + lrow, 2 * lhalf);      // half 0: group 2*lhalf
    const uint32_t xl1 = XR + tile_off(tokw * WM + lrow, 1 + 2 * lhalf);  // half 1: group 1 + 2*lhalf
    const uint32_t wl = WR + lrow * 16 + lhalf * 8;
    // fragments fm sit 32 rows (2 KB) apart with the same swizzle: (row >> 2) & 3 depends on row % 16 only
    auto read_x = [&](uint32_t addr, v4i (&x)[FM]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) x[fm] = *reinterpret_cast<const v4i *>(smem + addr + fm * 2048);
    };
    // packed weights of a step: dwords 2*lhalf and 2*lhalf+1 of each of the wave's rows
    auto read_w = [&](uint32_t addr, v2u (&w)[NA][FW]) {
#pragma unroll
        for (int mat = 0; mat < NA; ++mat)
#pragma unroll
            for (int fn = 0; fn < FW; ++fn)
                w[mat][fn] = *reinterpret_cast<const v2u *>(smem + addr + mat * W_PK + (FOFF + fn) * 512);
    };

    v16i acc[NA][FM][FW];
#pragma unroll
    for (int mat = 0; mat < NA; ++mat)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FW; ++fn)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mat][fm][fn][v] = 0;

    // Operands of both half steps from one packed fragment: with the two dwords
    // as one 64-bit value, one shift gives field i of both (the bits a shift
    // moves across the dword boundary fall outside the 0x03030303 mask).
    auto expand2 = [](v2u w, v4i &b0, v4i &b1) {
        constexpr uint32_t M = 0x03030303u;
        const uint64_t v = ((uint64_t)w.y << 32) | w.x;
        const uint64_t v2 = shr64<2>(v), v4 = shr64<4>(v), v6 = shr64<6>(v);
        b0 = v4i{(int)(w.x & M), (int)((uint32_t)v2 & M), (int)((uint32_t)v4 & M), (int)((uint32_t)v6 & M)};
        b1 = v4i{(int)(w.y & M), (int)((uint32_t)(v2 >> 32) & M), (int)((uint32_t)(v4 >> 32) & M),
                 (int)((uint32_t)(v6 >> 32) & M)};
    };
    // first half step: expands every fragment but the first (whose operands
    // were prepared before the barrier), keeping the second half's operands,
    // and runs the MFMAs of the first half as soon as each is ready
    auto mfma_half0_rest = [&](const v4i (&x)[FM], const v2u (&w)[NA][FW], v4i (&b1)[NA][FW]) {
#pragma unroll
        for (int mat = 0; mat < NA; ++mat)
#pragma unroll
            for (int fn = 0; fn < FW; ++fn) {
                if (mat == 0 && fn == 0) continue;
                v4i b0;
                expand2(w[mat][fn], b0, b1[mat][fn]);
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[mat][fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x[fm], b0, acc[mat][fm][fn], 0, 0, 0);
            }
    };
    auto mfma_half1 = [&](const v4i (&x)[FM], const v4i (&b1)[NA][FW]) {
#pragma unroll
        for (int mat = 0; mat < NA; ++mat)
#pragma unroll
            for (int fn = 0; fn < FW; ++fn)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
                    acc[mat][fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x[fm], b1[mat][fn], acc[mat][fm][fn], 0, 0, 0);
    };

    // prologue: the tile's per-token sum_k q and s (rows past m re-read the last
    // token), then stages 0..DB-1, all by direct loads; stages 0 and 1 landed
    if (wave * 64 < BM) {
        int64_t m = m0 + wave * 64 + lane;
        m = m < a.m ? m : a.m - 1;
        const uint32_t toff = (uint32_t)(m - m0) * 4;
        dma4(a.sumq + m0, toff, lds0 + TQ + wave * 256);
        if constexpr (EPI != EPI_ACC) dma4(a.s + m0, toff, lds0 + TS + wave * 256);
    }
    const int nst = nks / SPB;  // stages (SPB = 2 only for an even step count)
    for (int j = 0; j < DB; ++j)
        if (j < nst) dma_stage(j, j * XS, j * WS);
    if (DB < nst) ring_barrier<(DB - 2) * DPS>();
    else ring_barrier<0>();

    auto adv = [](uint32_t &o, uint32_t step, uint32_t end) {
        o += step;
        o = o >= end ? o - end : o;
    };

    v2u wA[NA][FW], wB[NA][FW];
    v4i x[FM];
    read_w(wl, wA);
    read_x(xl0, x);
    v4i p0, p1;  // both half-step operands of fragment (0, 0) of the coming step
    expand2(wA[0][0], p0, p1);

    // One 64-input step. Right after a barrier its first MFMAs start on
    // operands already in registers; the direct loads (issue), the reads of this
    // step's second activation half (ya) and of the next step's packed weights
    // (wa) go out in their shadow, the next step's first activation half (xa)
    // is read during the second half, and the next step's first expansion runs
    // last. The reads of the next step's data run unconditionally (straight-line
    // code keeps the compiler's LDS wait counts exact); in the last step they
    // read stages that are never used.
    auto step = [&](v2u (&wc)[NA][FW], v2u (&wn)[NA][FW], uint32_t ya, uint32_t wa, uint32_t xa, auto &&issue) {
        v4i b1[NA][FW];
        b1[0][0] = p1;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            acc[0][fm][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x[fm], p0, acc[0][fm][0], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue();
        v4i y[FM];
        read_x(ya, y);
        read_w(wa, wn);
        __builtin_amdgcn_sched_barrier(0);
        mfma_half0_rest(x, wc, b1);
        __builtin_amdgcn_sched_barrier(0);
        read_x(xa, x);
        __builtin_amdgcn_sched_barrier(0);
        mfma_half1(y, b1);
        expand2(wn[0][0], p0, p1);
    };

    // ring positions (byte offsets): the current and next stage of each ring and
    // the stages stage S+DB is loaded into
    uint32_t xs_cur = 0, xs_nxt = XS, ws_cur = 0, ws_nxt = WS;
    uint32_t xs_iss = (DB % SBX) * XS, ws_iss = (DB % SBW) * WS;
    auto advance = [&] {
        adv(xs_cur, XS, SBX * XS);
        adv(xs_nxt, XS, SBX * XS);
        adv(ws_cur, WS, SBW * WS);
        adv(ws_nxt, WS, SBW * WS);
        adv(xs_iss, XS, SBX * XS);
        adv(ws_iss, WS, SBW * WS);
    };
    // Before the barrier that ends stage S, stage S+2 must have landed: the
    // following stage reads (part of) it before its own barrier. The barrier
    // leaves the last FM LDS reads of the stage in flight: they fetch the first
    // activation half of the next step, which lives in a ring slot the coming
    // direct loads do not touch; every read of the slot those loads overwrite
    // was issued earlier and has completed.
    if constexpr (SPB == 1) {
        // one barrier per step; two steps per iteration so the packed-weight
        // registers alternate without copies; no branch inside the body (a merge
        // of the accumulators there costs register-class copies), the odd last
        // step runs after the loop
        auto one = [&](int ks, v2u (&wc)[NA][FW], v2u (&wn)[NA][FW]) {
            const bool issue = ks + DB < nks;
            step(wc, wn, xl1 + xs_cur, wl + ws_nxt, xl0 + xs_nxt, [&] {
                if (issue) dma_stage(ks + DB, xs_iss, ws_iss);
            });
            advance();
            if (issue) ring_barrier<VM_SLACK, FM>();
            else ring_barrier<0, FM>();
        };
        int ks = 0;
        for (; ks + 1 < nks; ks += 2) {
            one(ks, wA, wB);
            one(ks + 1, wB, wA);
        }
        if (ks < nks) one(ks, wA, wB);
    } else {
        // one barrier per pair of steps: the first step reads the second's
        // weights and first activation half from the same stage, the second
        // reads the next stage
        for (int S = 0; S < nst; ++S) {
            const bool issue = S + DB < nst;
            step(wA, wB, xl1 + xs_cur, wl + ws_cur + W_STAGE, xl0 + xs_cur + X_TILE, [&] {
                if (issue) dma_stage(S + DB, xs_iss, ws_iss);
            });
            step(wB, wA, xl1 + xs_cur + X_TILE, wl + ws_nxt, xl0 + xs_nxt, [] {});
            advance();
            if (issue) ring_barrier<VM_SLACK, FM>();
            else ring_barrier<0, FM>();
        }
    }

    // epilogue (the loop's last barrier made the per-token terms visible)
    store_tile<FM, FW, FOFF, EPI>(a, acc, reinterpret_cast<const int *>(smem + TQ),
                                  reinterpret_cast<const float *>(smem + TS), m0, n0, tokw, lrow, lhalf);
}

// WSPLIT = 1: four waves, each with all FN fragments; 2: eight waves, two per
// SIMD, splitting the fragments (gemm_waves)
template <int FM, int FN, int EPI, int DB, int SPB, int WSPLIT>
__global__ __launch_bounds__(256 * WSPLIT) void gemm_kernel(GemmArgs a)
{
    constexpr int BM = 128 * FM, BN = 32 * FN;
    extern __shared__ __align__(16) int8_t smem[];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // XCD-aware tile order: workgroups id, id+8, id+16, ... share an XCD and get
    // consecutive tiles, row-major over (m tile, n tile)
    const int tiles = a.n_tiles * a.m_tiles;
    const int id = blockIdx.x, xcd = id & 7, per = tiles >> 3, rem = tiles & 7;
    const int tile = xcd * per + min(xcd, rem) + (id >> 3);
    const int64_t m0 = (int64_t)(tile / a.n_tiles) * BM, n0 = (int64_t)(tile % a.n_tiles) * BN;

    if constexpr (WSPLIT == 1) {
        gemm_waves<FM, FN, EPI, DB, SPB, 4, FN, 0, true>(a, smem, wave, m0, n0);
    } else if constexpr (WSPLIT == 2) {
        constexpr int F0 = (FN + 1) / 2;
        if (wave < 4) gemm_waves<FM, FN, EPI, DB, SPB, 8, F0, 0, true>(a, smem, wave, m0, n0);
        else gemm_waves<FM, FN, EPI, DB, SPB, 8, FN - F0, F0, false>(a, smem, wave, m0, n0);
    } else {
        // sixteen waves, four per SIMD: fragment groups of F, F, F and FN - 3F
        constexpr int F = (FN + 3) / 4;
        static_assert(WSPLIT == 4 && FN > 3 * F, "four non-empty fragment groups");
        const int g = wave >> 2;
        if (g == 0) gemm_waves<FM, FN, EPI, DB, SPB, 16, F, 0, true>(a, smem, wave, m0, n0);
        else if (g == 1) gemm_waves<FM, FN, EPI, DB, SPB, 16, F, F, false>(a, smem, wave, m0, n0);
        else if (g == 2) gemm_waves<FM, FN, EPI, DB, SPB, 16, F, 2 * F, false>(a, smem, wave, m0, n0);
        else gemm_waves<FM, FN, EPI, DB, SPB, 16, FN - 3 * F, 3 * F, false>(a, smem, wave, m0, n0);
    }
}

// Eight waves (two per SIMD, the fragments split) except for the 128-token
// tiles of a gate/up pair: same-box A/B at 2048 tokens, eight waves took the
// prefill layers 48.6 / 47.5 against 51.1 / 50.2 us (256x224 and 128x160
// tiles) and the 8B gate/up pair's 256x128 tiles 356 against 367.5 us per FFN,
// but its 128x128 tiles 364.5 against 357 us
template <int FM, int FN, int EPI, int DB, int SPB = 1, int WSPLIT = (FM == 2 || EPI != EPI_GATE ? 2 : 1)>
static hipError_t launch_tile(GemmArgs a, hipStream_t st)
{
    constexpr int NA = EPI == EPI_GATE ? 2 : 1;
    constexpr size_t xs = (size_t)SPB * 128 * FM * 64, ws = (size_t)SPB * NA * 256 * 16;
    constexpr size_t lds = (size_t)(DB + 1) * xs + (size_t)(SPB == 1 ? DB : DB + 1) * ws + 2 * 128 * FM * 4;
    static_assert(lds <= 160 * 1024, "LDS budget");
    a.n_tiles = (int)ceil_div(a.n, 32 * FN);
    a.m_tiles = (int)ceil_div(a.m, 128 * FM);
    const auto kern = gemm_kernel<FM, FN, EPI, DB, SPB, WSPLIT>;
    static LdsLimit lim;
    if (hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(kern), (int)lds, lim)) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.n_tiles * a.m_tiles)), dim3(kThreads * WSPLIT), lds, st, a);
    return hipGetLastError();
}

// 128-token tiles of one matrix: two steps per stage when the step count is even
template <int FN, int EPI>
static hipError_t launch_fm1(const GemmArgs &a, hipStream_t st)
{
    if ((a.kp / 64) % 2 == 0) return launch_tile<1, FN, EPI, 3, 2>(a, st);
    return launch_tile<1, FN, EPI, 6, 1>(a, st);
}

// Tile shape: the (FM, FN) of least cost, rounds over the 256 CUs times a
// per-tile cost of FM*FN*NA MFMA blocks, the weight expansion (about 0.2 of
// a block per block on 128-token tiles, half that on 256-token tiles, which
// expand each operand once for two MFMAs: the gate/up pair at 2048 x 14336
// took 315 us on 128x192 tiles and 265 us on 256x128) and a fixed per-step
// overhead. Shapes are limited to those whose accumulators and operands fit
// the register file without spilling: at most 14 accumulator blocks for one
// matrix; for the gate/up pair 12 on 128-token tiles, or 256x128 (16 blocks:
// all 256 AGPRs and 256 VGPRs).
struct TileShape {
    int fm, fn;
    double cost;  // modelled time: rounds over the 256 CUs x per-tile cost
};
static bool tile_allowed(int fm, int fn, int na)
{
    if (na == 2) return (fm == 1 && fn >= 4 && fn <= 6) || (fm == 2 && (fn == 4 || fn == 2));
    return fn >= 4 && fm * fn <= 14;
}
static int64_t tile_count(int64_t m, int64_t n, int fm, int fn) { return ceil_div(n, 32 * fn) * ceil_div(m, 128 * fm); }
static TileShape pick_tile(int64_t m, int64_t n, int na)
{
    TileShape best{1, 4, 1e300};
    for (int fm = 2; fm >= 1; --fm)
        for (int fn = 8; fn >= 2; --fn) {
            if (!tile_allowed(fm, fn, na)) continue;
            const int64_t rounds = ceil_div(tile_count(m, n, fm, fn), 256);
            const double cost = (double)rounds * (fm * fn * na * (1.0 + 0.2 / fm) + 3.0);
            if (cost < best.cost) best = TileShape{fm, fn, cost};
        }
    return best;
}

// Output columns given to a second launch. When the best tiling leaves its last
// round over the 256 CUs at most half full (the 8B gate/up pair at 2048 tokens:
// 896 tiles of 256x128, 3.5 rounds), the columns of the full rounds keep that
// tiling and the rest run as a launch of their own, whose smaller tiles spread
// over all CUs (there: 12288 + 2048 columns, the latter as 256 tiles of 128x128).
// Returns the column count of the first launch, or n for one launch. The
// modelled cost adds one block-cost unit per extra launch.
static int64_t split_columns(int64_t m, int64_t n, int na)
{
    const TileShape t = pick_tile(m, n, na);
    const int64_t tiles = tile_count(m, n, t.fm, t.fn), last = tiles % 256;
    if (tiles <= 256 || last == 0 || last > 128) return n;
    const int64_t m_tiles = ceil_div(m, 128 * t.fm);
    const int64_t n_main = (tiles / 256) * 256 / m_tiles * (32 * t.fn);
    if (n_main <= 0 || n_main >= n) return n;
    const double split = pick_tile(m, n_main, na).cost + pick_tile(m, n - n_main, na).cost + 1.0;
    return split < t.cost ? n_main : n;
}

// 256x224 tiles run sixteen waves, four per SIMD, in fragment groups of 2, 2,
// 2 and 1 (same-box A/B, prefill 2560->6912 layer at 2048 tokens: 46.7
// against 48.6 us with eight waves); 256x128 tiles keep eight (sixteen: the
// 8B FFN at 2048 tokens 379-387 against 360-366 us).
// Ring depths (stages requested ahead): with eight waves per workgroup the
// shallower rings measured faster (same-box A/B at 2048 tokens: prefill step
// 0.0940 against 0.0955 ms with DB 4 / 3 instead of 6 / 5; 8B FFN 351.5
// against 353 us with DB 4 instead of 5 and 6)
template <int EPI>
static hipError_t launch_epi(const GemmArgs &a, hipStream_t st)
{
    constexpr int NA = EPI == EPI_GATE ? 2 : 1;
    const TileShape t = pick_tile(a.m, a.n, NA);
    if constexpr (NA == 1) {
        if (t.fm == 2) {
            switch (t.fn) {
            case 4: return launch_tile<2, 4, EPI, 4>(a, st);
            case 5: return launch_tile<2, 5, EPI, 4>(a, st);
            case 6: return launch_tile<2, 6, EPI, 4>(a, st);
            default: return launch_tile<2, 7, EPI, 4, 1, 4>(a, st);  // sixteen waves
            }
        }
        switch (t.fn) {
        case 4: return launch_fm1<4, EPI>(a, st);
        case 5: return launch_fm1<5, EPI>(a, st);
        case 6: return launch_fm1<6, EPI>(a, st);
        case 7: return launch_fm1<7, EPI>(a, st);
        default: return launch_fm1<8, EPI>(a, st);
        }
    } else {
        if (t.fm == 2) {  // 114 KB of LDS
            if (t.fn == 2) return launch_tile<2, 2, EPI, 4>(a, st);
            return launch_tile<2, 4, EPI, 4>(a, st);
        }
        switch (t.fn) {
        case 4: return launch_tile<1, 4, EPI, 8>(a, st);
        case 5: return launch_tile<1, 5, EPI, 8>(a, st);
        default: return launch_tile<1, 6, EPI, 8>(a, st);
        }
    }
}

hipError_t launch_gemm(const GemmProblem &p, hipStream_t st)
{
    GemmArgs a;
    a.qp = p.qp; a.kp = p.kp; a.s = p.s; a.sumq = p.sumq; a.m = p.m; a.n = p.n;
    a.w0 = p.w0; a.w1 = p.w1; a.ldw = p.ldw; a.gamma0 = p.gamma0; a.gamma1 = p.gamma1;
    a.out = p.out; a.acc_out = p.acc_out; a.ldo = p.n; a.qmax = p.qmax;
    a.n_tiles = a.m_tiles = 0;
    auto run = [&](const GemmArgs &g) {
        switch (p.epi) {
        case EPI_Y: return launch_epi<EPI_Y>(g, st);
        case EPI_ACC: return launch_epi<EPI_ACC>(g, st);
        default: return launch_epi<EPI_GATE>(g, st);
        }
    };
    const int64_t n_main = split_columns(p.m, p.n, p.epi == EPI_GATE ? 2 : 1);
    if (n_main == p.n) return run(a);
    // columns [0, n_main) and [n_main, n): weight rows and output columns offset,
    // output row stride unchanged
    GemmArgs b = a;
    a.n = n_main;
    b.n = p.n - n_main;
    b.w0 = p.w0 + n_main * p.ldw;
    if (p.w1) b.w1 = p.w1 + n_main * p.ldw;
    if (p.out) b.out = p.out + n_main;
    if (p.acc_out) b.acc_out = p.acc_out + n_main;
    if (hipError_t e = run(a)) return e;
    return run(b);
}

}  // namespace bl
