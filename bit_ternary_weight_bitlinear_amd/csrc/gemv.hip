// gemv.hip -- decode-time BitLinear (m <= 4 tokens) for gfx950.
//
// The W1.58A8 product ("穿越1比特的奇幻旅程", section 推理实现 / GPU端) at small m is a
// stream over the packed weights: 2 bits per weight is the whole HBM traffic.
// Design:
//  * one workgroup per CU: workgroup b owns rows [b*R, b*R + R) with
//    R = ceil(n / 256), a contiguous block of R * k/4 bytes. Each row is cut
//    into blocks of eight 16-byte chunks (512 weights); a group of 8 lanes
//    takes one (row, block) unit and each lane one chunk, so every group reads
//    128 contiguous bytes and a wave's 8 groups read the same block of 8 rows
//    (the activation chunks they need are then shared: LDS broadcast). Units
//    go to the 64 groups round-robin, row index fastest. Every CU reads the
//    same number of bytes and does the activation quantization below once;
//  * each thread first issues its activation loads, then all of its weight
//    loads (a compile-time count, no branches), so everything is in flight at
//    once and the quantization can start as soon as the activations arrive;
//  * the workgroup quantizes the m tokens itself (absmax with DPP wave
//    reductions, round by the 1.5*2^23 add) into LDS in the qperm order: no
//    separate activation kernel, no launch gap;
//  * codes are decoded in registers with four AND masks and one shift per
//    dword (code<<0, <<2, <<4 and, after a right shift by one, <<5 -- each fits a
//    signed byte) and fed to v_dot4_i32_i8 against the qperm dwords; the four
//    partial sums are brought back to scale by exact shifts;
//  * the 8 lane sums of a unit are added with DPP inside the group, and one
//    lane adds the unit's sum into its row's int32 accumulator in LDS
//    (ds_add_u32); integer sums are exact, so the order of the adds does not
//    matter and the result is deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kNumCUs = 256;          // MI355X: 8 XCDs x 32 CUs
constexpr int kMaxUnits = 1024;       // (row, 8-chunk block) units per workgroup and matrix
constexpr int kGemvLdsLimit = 60 * 1024;
constexpr int kSlots = 4;             // at most this many activation groups per thread in registers
constexpr int kGT = 512;              // threads per workgroup (8 waves: two per SIMD)
constexpr int kGW = kGT / 64;         // waves per workgroup

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
    float *hmax_part;   // gate/up pair only, optional: max |h| per (workgroup, token)
    const float *pre_s;       // PREQ: the quantization kernel's scales and code sums
    const int32_t *pre_sumq;
    float qmax;               // code of the largest magnitude (127; 12 for doubled E2M1 codes)
    int rows_per_wg;  // R
    int chunks;       // kp / 64
    const float *gain;  // NORM: per-input gain [k], or NULL (last: the other fields keep their offsets)
    int keep;           // A4: entries kept per token
};

// LDS slot of activation group (c, d): 16-byte slots rotated by (c >> 2) & 3 so
// that lanes reading neighbouring chunks spread over the banks.
__device__ inline int lds_slot(int c, int d) { return c * 64 + ((d ^ ((c >> 2) & 3)) << 4); }

// RES: all m*ceil(k/16) activation groups fit in SL <= kSlots per thread
// (loaded once, quantized from registers; SL is sized to the problem so that
// unused slots hold no registers). FULL: k % 16 == 0. JM: (row, 8-chunk block)
// units per lane group. PREQ: x holds quantized rows [m][kp] in the qperm
// order (with pre_s and pre_sumq) written by a quantization kernel: their
// 16-byte words go to LDS as they are, one barrier, no quantization.
// NORM: one token whose activations are first RMS-normalized (subln): x^ =
// (x * r) * g with r = 1 / sqrt(fp32(S / k) + 1e-5), S = sum x^2 as an fp64
// double-double sum over the workgroup, g the optional per-input gain (none:
// x^ = x * r); then the same quantization and product.
// A4: one token quantized to 4-bit E2M1 codes instead (the a.keep largest
// |x| kept, v = x * (6 / s) to the nearest E2M1 value, stored doubled): tau,
// the keep-th largest |x|, by a radix select over the workgroup (two 11-bit
// digit passes for bf16, histograms in LDS), the same select as the 4-bit
// quantization kernel, so the codes are the same.
template <typename T, int MT, bool DUAL, bool RES, bool FULL, int JM, int SL = kSlots, bool PREQ = false,
          bool NORM = false, bool A4 = false>
__global__ __launch_bounds__(512) void gemv_kernel(GemvArgs a)
{
    static_assert(!PREQ || (RES && FULL && !DUAL), "quantized rows: resident slots, one matrix");
    static_assert(!NORM || (RES && FULL && !DUAL && !PREQ && MT == 1), "normalized decode: one token, one matrix");
    static_assert(!A4 || (RES && FULL && !DUAL && !PREQ && MT == 1 && !NORM && sizeof(T) == 2),
                  "4-bit decode: one bf16 token, one matrix");
    constexpr int NA = DUAL ? 2 : 1;
    extern __shared__ __align__(16) int8_t lds[];  // q [MT][kp], then int32 sums [NA][MT][R]
    __shared__ float red_f[MT][kGW];
    __shared__ int red_i[MT][kGW];
    int8_t *q_lds = lds;
    int *acc_lds = reinterpret_cast<int *>(lds + MT * a.kp);

    // the scalars of the later phases are requested here, before the
    // activation loads: fetched where they are used, the kernel-argument line
    // with the output pointers missed the scalar cache inside the quantization
    // and gamma took an L2 round trip between the last barrier and the stores
    const float g0 = a.gamma0[0];
    const float g1 = DUAL ? a.gamma1[0] : 0.0f;
    float pre_st[MT];
    int pre_sq[MT];
    if constexpr (PREQ) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            pre_st[t] = a.pre_s[t];
            pre_sq[t] = a.pre_sumq[t];
        }
    }
    asm volatile("" ::"s"(a.out), "s"(a.acc_out), "s"(a.q_out), "s"(a.s_out), "s"(a.hmax_part), "s"(a.qmax));

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int R = a.rows_per_wg, C = a.chunks;
    const int64_t r0 = (int64_t)blockIdx.x * R;
    const int rows = (int)((a.n - r0) < R ? (a.n - r0) : R);
    const T *x = static_cast<const T *>(a.x);
    const int GP = (int)(a.kp / 16);
    const int G = PREQ ? GP : (int)ceil_div(a.k, 16);  // quantized rows include their zero padding
    const int NG = MT * G;

    // 1. activation loads first: the quantization waits only for these. They
    //    are kept as raw words and, for a small weight share per thread,
    //    converted only after the weight loads are issued, so both are in
    //    flight together. With a large share (6 or more 16-byte loads, the 8B
    //    FFN matrices) the activations are converted, i.e. waited for, before
    //    the weights are requested: otherwise they queue behind the weights
    //    and the quantization ends later (measured: ~0.3 us per launch either
    //    way). Every slot is loaded (clamped to a valid group), with no branch.
    constexpr bool kActFirst = JM * NA >= 6 && !PREQ;
    constexpr int XQ = PREQ ? 1 : (int)sizeof(T);  // 16-byte words per 16-input group (bf16: 2, fp32: 4)
    uint4 xq[SL][XQ];
    int slot_t[SL], slot_g[SL];
    if constexpr (RES) {
#pragma unroll
        for (int s = 0; s < SL; ++s) {
            const int f = min(tid + s * kGT, NG - 1);
            slot_t[s] = MT == 1 ? 0 : f / G;
            slot_g[s] = f - slot_t[s] * G;
            const uint4 *p = PREQ ? reinterpret_cast<const uint4 *>(static_cast<const int8_t *>(a.x) +
                                                                    slot_t[s] * a.kp + 16 * (int64_t)slot_g[s])
                                  : reinterpret_cast<const uint4 *>(x + slot_t[s] * a.k + 16 * (int64_t)slot_g[s]);
#pragma unroll
            for (int q = 0; q < XQ; ++q) xq[s][q] = p[q];
        }
    }
    // the gain entries of the slots' inputs, requested with the activations
    float4 gq[NORM ? SL : 1][4];
    if constexpr (NORM) {
        if (a.gain) {
#pragma unroll
            for (int s = 0; s < SL; ++s) {
                const float4 *gp = reinterpret_cast<const float4 *>(a.gain + 16 * (int64_t)slot_g[s]);
#pragma unroll
                for (int j = 0; j < 4; ++j) gq[s][j] = gp[j];
            }
        }
    }
    float xr[SL][16];
    if constexpr (RES && kActFirst) {
        // only the activation loads are outstanding here
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int s = 0; s < SL; ++s) unpack_group<T>(xq[s], xr[s]);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. the weight units of this thread: unit u = group + 64*j is (row u % rows,
    //    block u / rows); lane l of the group takes chunk 8*block + l. Lanes past
    //    the row's last chunk (and whole units past the end) re-read chunk C-1 of
    //    a row of this workgroup; their sums are dropped.
    const int grp = tid >> 3, li = tid & 7;
    int tr[JM], tc[JM];
    bool tv[JM];
    {
        const int db = (kGT / 8) / rows, dr = (kGT / 8) - db * rows;
        int b = grp / rows;
        int r = grp - b * rows;
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int c = 8 * b + li;
            tv[j] = c < C;
            tr[j] = r;
            tc[j] = c < C ? c : C - 1;
            r += dr;
            b += db;
            if (r >= rows) {
                r -= rows;
                b += 1;
            }
        }
    }
    const int nunit = rows * ((C + 7) >> 3);
    // every slot is loaded, with no branch between the loads, so the waits
    // below can count them and the products of a unit start when its own
    // weights have arrived
    uint4 wa[JM], wb[JM];
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        const int64_t off = (r0 + tr[j]) * a.ldw + (int64_t)tc[j] * 16;
        wa[j] = load_nt16(a.w0 + off);
        if constexpr (DUAL) wb[j] = load_nt16(a.w1 + off);
    }
    // keep every load above this point in issue order: nothing below may be
    // hoisted between them, so all of this thread's reads are in flight at once
    __builtin_amdgcn_sched_barrier(0);
    // gamma is needed from here on (it has long arrived): without this use the
    // load sinks to the first barrier, whose wait then includes its latency
    asm volatile("" ::"s"(g0), "s"(g1));

    // 3. per-token absmax, then int8 codes into LDS in the qperm order
    if constexpr (RES && !kActFirst && !PREQ) {
#pragma unroll
        for (int s = 0; s < SL; ++s) unpack_group<T>(xq[s], xr[s]);
    }
    float st[MT], inv[MT];
    int sq[MT];
    if constexpr (PREQ) {
        // the quantized rows' words into LDS, their scales and sums from memory
#pragma unroll
        for (int s = 0; s < SL; ++s)
            if (tid + s * kGT < NG)
                *reinterpret_cast<uint4 *>(q_lds + slot_t[s] * a.kp + lds_slot(slot_g[s] >> 2, slot_g[s] & 3)) =
                    xq[s][0];
        for (int i = tid; i < NA * MT * R; i += kGT) acc_lds[i] = 0;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            st[t] = pre_st[t];
            inv[t] = 0.0f;
            sq[t] = pre_sq[t];
        }
        __syncthreads();
    } else {
        if constexpr (NORM) {
            // S over this thread's groups (slots past the last group re-read
            // it and are skipped here), then over the workgroup
            __shared__ double red_d[2 * kGW];
            double hi = 0.0, lo = 0.0;
#pragma unroll
            for (int s = 0; s < SL; ++s)
                if (tid + s * kGT < NG) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) dd_add(hi, lo, (double)xr[s][j] * (double)xr[s][j]);
                }
            const float r = norm_factor(block_sum_dd<kGW>(hi, lo, red_d), a.k);
            const bool has_gain = a.gain != nullptr;
#pragma unroll
            for (int s = 0; s < SL; ++s) {
#pragma unroll
                for (int j = 0; j < 16; ++j) xr[s][j] = xr[s][j] * r;
                if (has_gain) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        xr[s][4 * j + 0] = xr[s][4 * j + 0] * gq[s][j].x;
                        xr[s][4 * j + 1] = xr[s][4 * j + 1] * gq[s][j].y;
                        xr[s][4 * j + 2] = xr[s][4 * j + 2] * gq[s][j].z;
                        xr[s][4 * j + 3] = xr[s][4 * j + 3] * gq[s][j].w;
                    }
                }
            }
        }
        // 4-bit: the select's histograms, zeroed here and published by the
        // absmax barrier below (bf16: bits 30..20, then 19..16)
        constexpr int kA4Passes = 2;
        int *hist = nullptr;  // [kA4Passes][kDigitBins]
        if constexpr (A4) {
            __shared__ __align__(16) int hist_lds[kA4Passes * kDigitBins];
            hist = hist_lds;
            for (int i = tid; i < kA4Passes * kDigitBins / 4; i += kGT)
                reinterpret_cast<int4 *>(hist)[i] = make_int4(0, 0, 0, 0);
        }
        float amax[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) amax[t] = 0.0f;
        if constexpr (RES) {
#pragma unroll
            for (int s = 0; s < SL; ++s) {
                if (s * kGT < NG) {
                    float m = 0.0f;
#pragma unroll
                    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(xr[s][j]));
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        if (slot_t[s] == t) amax[t] = fmaxf(amax[t], m);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < MT; ++t)
                for (int g = tid; g < G; g += kGT) {
                    float f[16];
                    load_group<T, FULL>(x + t * a.k, a.k, g, f);
#pragma unroll
                    for (int j = 0; j < 16; ++j) amax[t] = fmaxf(amax[t], fabsf(f[j]));
                }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            amax[t] = wave_max(amax[t]);
            if (lane == 0) red_f[t][wave] = amax[t];
        }
        __syncthreads();
        int qs[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float mx = red_f[t][0];
#pragma unroll
            for (int w = 1; w < kGW; ++w) mx = fmaxf(mx, red_f[t][w]);
            st[t] = fmaxf(mx, kEps);
            inv[t] = (A4 ? 6.0f : 127.0f) / st[t];
            qs[t] = 0;
        }
        uint32_t tau = 0;  // 4-bit: the keep-th largest |x| (as bits)
        if constexpr (A4) {
            uint32_t prefix = 0, pmask = 0;
            int want = a.keep;
#pragma unroll
            for (int p = 0; p < kA4Passes; ++p) {
                const int hi = 31 - p * kDigitBits;
                const int lo = hi - kDigitBits > 16 ? hi - kDigitBits : 16;
                const uint32_t dmask = (1u << (hi - lo)) - 1u;
                int *h = hist + p * kDigitBins;
#pragma unroll
                for (int s = 0; s < SL; ++s)
                    if (tid + s * kGT < NG) {  // slots past the last group re-read it: not counted
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const uint32_t key = __float_as_uint(fabsf(xr[s][j]));
                            if ((key & pmask) == prefix) atomicAdd(&h[(key >> lo) & dmask], 1);
                        }
                    }
                __syncthreads();
                prefix |= pick_digit(h, want) << lo;
                pmask |= dmask << lo;
            }
            tau = prefix;
        }
        auto emit = [&](int t, int g, const float f[16], float iv) {
            uint4 pv, nv;
            int sum;
            if constexpr (A4) {
                int qi[16];
                sum = 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    qi[j] = __float_as_uint(fabsf(f[j])) >= tau ? e2m1_doubled(f[j] * iv) : 0;
                    sum += qi[j];
                }
                pv = qperm_pack(qi);
                nv = make_uint4(0, 0, 0, 0);  // no natural-order copy (q_out is not used in this mode)
            } else {
                sum = quant_group(f, iv, &pv, &nv);
            }
#pragma unroll
            for (int u = 0; u < MT; ++u)
                if (u == t) qs[u] += sum;
            *reinterpret_cast<uint4 *>(q_lds + t * a.kp + lds_slot(g >> 2, g & 3)) = pv;
            if (a.q_out && blockIdx.x == 0) {
                const uint32_t dw[4] = {nv.x, nv.y, nv.z, nv.w};
                uint32_t *dst = reinterpret_cast<uint32_t *>(a.q_out + t * a.k + 16 * (int64_t)g);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (16 * (int64_t)g + 4 * j < a.k) dst[j] = dw[j];
            }
        };
        if constexpr (RES) {
#pragma unroll
            for (int s = 0; s < SL; ++s) {
                if (tid + s * kGT < NG) {
                    float iv = inv[0];
#pragma unroll
                    for (int t = 1; t < MT; ++t)
                        if (slot_t[s] == t) iv = inv[t];
                    emit(slot_t[s], slot_g[s], xr[s], iv);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < MT; ++t)
                for (int g = tid; g < G; g += kGT) {
                    float f[16];
                    load_group<T, FULL>(x + t * a.k, a.k, g, f);
                    emit(t, g, f, inv[t]);
                }
        }
        // zero inputs of the padding up to kp, and the row accumulators
#pragma unroll
        for (int t = 0; t < MT; ++t)
            for (int g = G + tid; g < GP; g += kGT)
                *reinterpret_cast<uint4 *>(q_lds + t * a.kp + lds_slot(g >> 2, g & 3)) = make_uint4(0, 0, 0, 0);
        for (int i = tid; i < NA * MT * R; i += kGT) acc_lds[i] = 0;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            qs[t] = wave_sum(qs[t]);
            if (lane == 0) red_i[t][wave] = qs[t];
            if (a.s_out && blockIdx.x == 0 && tid == 0) a.s_out[t] = st[t];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            sq[t] = 0;
#pragma unroll
            for (int w = 0; w < kGW; ++w) sq[t] += red_i[t][w];
        }
    }

    // 4. decode the 2-bit codes in registers, v_dot4 against the qperm dwords,
    //    sum each unit over its 8 lanes and add it into its row's LDS accumulator
#pragma unroll
    for (int j = 0; j < JM; ++j) {
        // uniform per wave: the wave's first unit of this round exists
        if (wave * 8 + j * (kGT / 8) < nunit) {
            const int c = tc[j];
            int acc[MT][4], accb[MT][4];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[t][i] = accb[t][i] = 0;
            const uint32_t wda[4] = {wa[j].x, wa[j].y, wa[j].z, wa[j].w};
            uint32_t wdb[4] = {0, 0, 0, 0};
            if constexpr (DUAL) {
                wdb[0] = wb[j].x;
                wdb[1] = wb[j].y;
                wdb[2] = wb[j].z;
                wdb[3] = wb[j].w;
            }
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
            // lane 0 of the group holds chunk 8*block, so its flag says whether
            // the unit exists
            const bool add = li == 0 && tv[j];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                // undo the field shifts (each partial is an exact multiple)
                int va = acc[t][0] + (acc[t][1] >> 2) + (acc[t][2] >> 4) + (acc[t][3] >> 5);
                va = group8_sum(tv[j] ? va : 0);
                if (add) atomicAdd(&acc_lds[t * R + tr[j]], va);
                if constexpr (DUAL) {
                    int vb = accb[t][0] + (accb[t][1] >> 2) + (accb[t][2] >> 4) + (accb[t][3] >> 5);
                    vb = group8_sum(tv[j] ? vb : 0);
                    if (add) atomicAdd(&acc_lds[(MT + t) * R + tr[j]], vb);
                }
            }
        }
    }
    __syncthreads();

    // 5. rescale: y = (float)acc * ((s / 127) * gamma); the pair gives h = relu(g)^2 * u
    float hmax[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const float ca = token_scale(st[t], g0, a.qmax);
        const float cb = DUAL ? token_scale(st[t], g1, a.qmax) : 0.0f;
        hmax[t] = 0.0f;
        for (int r = tid; r < rows; r += kGT) {
            const int va = acc_lds[t * R + r] - sq[t];
            const float ya = (float)va * ca;
            float *o = a.out + t * a.n + r0 + r;
            if constexpr (DUAL) {
                const int vb = acc_lds[(MT + t) * R + r] - sq[t];
                const float h = sq_relu_gate(ya, (float)vb * cb);
                *o = h;
                hmax[t] = fmaxf(hmax[t], fabsf(h));
            } else {
                *o = ya;
                if (a.acc_out) a.acc_out[t * a.n + r0 + r] = va;
            }
        }
    }
    if constexpr (DUAL) {
        // the requantization's absmax, one partial per workgroup and token
        if (a.hmax_part) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float mw = wave_max(hmax[t]);
                if (lane == 0) red_f[t][wave] = mw;
            }
            __syncthreads();
            if (tid < MT) {
                float mx = 0.0f;
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    if (t == tid)
#pragma unroll
                        for (int w = 0; w < kGW; ++w) mx = fmaxf(mx, red_f[t][w]);
                a.hmax_part[(int64_t)blockIdx.x * MT + tid] = mx;
            }
        }
    }
}

// ---------------------------------------------------------------- host side

// Rows per workgroup: one workgroup per CU while that keeps each thread at
// about 8 weight loads or fewer (counting both matrices of a gate/up pair);
// larger matrices are split further so more workgroups share a CU. Fewer,
// larger workgroups repeat the activation prologue less often: with at most
// 4 loads per thread the 8B FFN at one token took ~0.4 us longer.
constexpr int kTargetLoads = 8;

// (row, 8-chunk block) units per row, and the most rows a workgroup may own
static int64_t gemv_blocks(int64_t chunks) { return ceil_div(chunks, (int64_t)8); }
static int64_t gemv_rows_max(int64_t chunks) { return kMaxUnits / gemv_blocks(chunks); }

static int64_t gemv_rows_per_wg(int64_t n, int64_t chunks, bool dual)
{
    int64_t r = ceil_div(n, kNumCUs);
    const int64_t na = dual ? 2 : 1;
    while (r > 1 && r * chunks * na > (int64_t)kTargetLoads * kGT) r = ceil_div(r, 2);
    const int64_t rmax = gemv_rows_max(chunks);  // units per workgroup <= kMaxUnits
    if (r > rmax) r = rmax;
    return r < 1 ? 1 : r;
}

static size_t gemv_lds_bytes(int64_t m, int64_t kp, int64_t r, bool dual)
{
    return (size_t)(m * kp + (dual ? 2 : 1) * m * r * 4);
}

bool gemv_supported(int64_t m, int64_t kp)
{
    const int64_t chunks = kp / 64;
    if (m < 1 || m > 4 || gemv_blocks(chunks) > kMaxUnits) return false;
    // worst case over n: the most rows a workgroup may own
    const int64_t rmax = gemv_rows_max(chunks);
    return gemv_lds_bytes(m, kp, rmax, true) <= (size_t)kGemvLdsLimit;
}

namespace {

template <typename T, int MT, bool DUAL, bool RES, bool FULL, int JM, int SL = kSlots, bool PREQ = false,
          bool NORM = false, bool A4 = false>
void launch_one(dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    hipLaunchKernelGGL((gemv_kernel<T, MT, DUAL, RES, FULL, JM, SL, PREQ, NORM, A4>), grid, dim3(kGT), lds, st, a);
}

// one bf16 token, quantized to 4-bit E2M1 codes in the prologue
template <int SL>
void launch_a4(int jm, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    if (jm <= 1) launch_one<bf16_t, 1, false, true, true, 1, SL, false, false, true>(grid, lds, st, a);
    else if (jm <= 2) launch_one<bf16_t, 1, false, true, true, 2, SL, false, false, true>(grid, lds, st, a);
    else if (jm <= 3) launch_one<bf16_t, 1, false, true, true, 3, SL, false, false, true>(grid, lds, st, a);
    else if (jm <= 4) launch_one<bf16_t, 1, false, true, true, 4, SL, false, false, true>(grid, lds, st, a);
    else if (jm <= 6) launch_one<bf16_t, 1, false, true, true, 6, SL, false, false, true>(grid, lds, st, a);
    else if (jm <= 8) launch_one<bf16_t, 1, false, true, true, 8, SL, false, false, true>(grid, lds, st, a);
    else launch_one<bf16_t, 1, false, true, true, 16, SL, false, false, true>(grid, lds, st, a);
}

// one bf16 token, RMS-normalized in the prologue
template <int SL>
void launch_norm(int jm, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    if (jm <= 1) launch_one<bf16_t, 1, false, true, true, 1, SL, false, true>(grid, lds, st, a);
    else if (jm <= 2) launch_one<bf16_t, 1, false, true, true, 2, SL, false, true>(grid, lds, st, a);
    else if (jm <= 3) launch_one<bf16_t, 1, false, true, true, 3, SL, false, true>(grid, lds, st, a);
    else if (jm <= 4) launch_one<bf16_t, 1, false, true, true, 4, SL, false, true>(grid, lds, st, a);
    else if (jm <= 6) launch_one<bf16_t, 1, false, true, true, 6, SL, false, true>(grid, lds, st, a);
    else if (jm <= 8) launch_one<bf16_t, 1, false, true, true, 8, SL, false, true>(grid, lds, st, a);
    else launch_one<bf16_t, 1, false, true, true, 16, SL, false, true>(grid, lds, st, a);
}

// single token, whole groups, activations resident: the decode hot path, with
// the task count per thread matched closely
template <typename T, bool DUAL, int SL>
void launch_m1(int jm, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    if (jm <= 1) launch_one<T, 1, DUAL, true, true, 1, SL>(grid, lds, st, a);
    else if (jm <= 2) launch_one<T, 1, DUAL, true, true, 2, SL>(grid, lds, st, a);
    else if (jm <= 3) launch_one<T, 1, DUAL, true, true, 3, SL>(grid, lds, st, a);
    else if (jm <= 4) launch_one<T, 1, DUAL, true, true, 4, SL>(grid, lds, st, a);
    else if (jm <= 5) launch_one<T, 1, DUAL, true, true, 5, SL>(grid, lds, st, a);
    else if (jm <= 6) launch_one<T, 1, DUAL, true, true, 6, SL>(grid, lds, st, a);
    else if (jm <= 8) launch_one<T, 1, DUAL, true, true, 8, SL>(grid, lds, st, a);
    else if (jm <= 10) launch_one<T, 1, DUAL, true, true, 10, SL>(grid, lds, st, a);
    else if (jm <= 12) launch_one<T, 1, DUAL, true, true, 12, SL>(grid, lds, st, a);
    else if (jm <= 14) launch_one<T, 1, DUAL, true, true, 14, SL>(grid, lds, st, a);
    else launch_one<T, 1, DUAL, true, true, 16, SL>(grid, lds, st, a);
}

// 2..4 tokens, whole groups, activations resident
template <typename T, int MT, bool DUAL, int SL>
void launch_mt(int jm, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    if (jm <= 4) launch_one<T, MT, DUAL, true, true, 4, SL>(grid, lds, st, a);
    else if (jm <= 8) launch_one<T, MT, DUAL, true, true, 8, SL>(grid, lds, st, a);
    else launch_one<T, MT, DUAL, true, true, 16, SL>(grid, lds, st, a);
}

template <typename T, bool DUAL, int SL>
void launch_res(int m, int jm, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    switch (m) {
    case 1: launch_m1<T, DUAL, SL>(jm, grid, lds, st, a); break;
    case 2: launch_mt<T, 2, DUAL, SL>(jm, grid, lds, st, a); break;
    case 3: launch_mt<T, 3, DUAL, SL>(jm, grid, lds, st, a); break;
    default: launch_mt<T, 4, DUAL, SL>(jm, grid, lds, st, a); break;
    }
}

// anything else (k % 16 != 0, or activations too long for registers)
template <typename T, bool DUAL>
void launch_generic(int mt, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    switch (mt) {
    case 1: launch_one<T, 1, DUAL, false, false, 16>(grid, lds, st, a); break;
    case 2: launch_one<T, 2, DUAL, false, false, 16>(grid, lds, st, a); break;
    case 3: launch_one<T, 3, DUAL, false, false, 16>(grid, lds, st, a); break;
    default: launch_one<T, 4, DUAL, false, false, 16>(grid, lds, st, a); break;
    }
}

template <typename T, bool DUAL>
void dispatch(const GemvProblem &p, int jm, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    const bool res = p.m * ceil_div(p.k, 16) <= (int64_t)kSlots * kGT;
    const bool full = p.k % 16 == 0;
    if (!res || !full) {
        launch_generic<T, DUAL>((int)p.m, grid, lds, st, a);
        return;
    }
    // resident activation slots per thread: 1, 2 or 4
    const int64_t sl = ceil_div(p.m * ceil_div(p.k, 16), (int64_t)kGT);
    if (sl <= 1) launch_res<T, DUAL, 1>((int)p.m, jm, grid, lds, st, a);
    else if (sl <= 2) launch_res<T, DUAL, 2>((int)p.m, jm, grid, lds, st, a);
    else launch_res<T, DUAL, 4>((int)p.m, jm, grid, lds, st, a);
}

}  // namespace

int64_t gemv_grid(int64_t n, int64_t kp, bool dual)
{
    return ceil_div(n, gemv_rows_per_wg(n, kp / 64, dual));
}

bool gemv_prequant_supported(int64_t m, int64_t kp)
{
    return gemv_supported(m, kp) && m * (kp / 16) <= (int64_t)kSlots * kGT;
}

bool gemv_token_prologue_supported(int64_t m, int64_t k, bool bf16)
{
    return m == 1 && bf16 && k % 16 == 0 && gemv_supported(1, round_up(k, 64)) && k / 16 <= (int64_t)kSlots * kGT;
}

namespace {

template <int MT, int SL>
void launch_preq_mt(int jm, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    if (jm <= 2) launch_one<int8_t, MT, false, true, true, 2, SL, true>(grid, lds, st, a);
    else if (jm <= 4) launch_one<int8_t, MT, false, true, true, 4, SL, true>(grid, lds, st, a);
    else if (jm <= 8) launch_one<int8_t, MT, false, true, true, 8, SL, true>(grid, lds, st, a);
    else launch_one<int8_t, MT, false, true, true, 16, SL, true>(grid, lds, st, a);
}

template <int SL>
void launch_preq(int m, int jm, dim3 grid, size_t lds, hipStream_t st, const GemvArgs &a)
{
    switch (m) {
    case 1: launch_preq_mt<1, SL>(jm, grid, lds, st, a); break;
    case 2: launch_preq_mt<2, SL>(jm, grid, lds, st, a); break;
    case 3: launch_preq_mt<3, SL>(jm, grid, lds, st, a); break;
    default: launch_preq_mt<4, SL>(jm, grid, lds, st, a); break;
    }
}

}  // namespace

hipError_t launch_gemv(const GemvProblem &p, hipStream_t st)
{
    GemvArgs a;
    a.x = p.x; a.k = p.k; a.kp = p.kp; a.n = p.n;
    a.w0 = p.w0; a.w1 = p.w1; a.ldw = p.ldw;
    a.gamma0 = p.gamma0; a.gamma1 = p.gamma1;
    a.out = p.out; a.acc_out = p.acc_out; a.q_out = p.q_out; a.s_out = p.s_out;
    a.hmax_part = p.hmax_part; a.pre_s = p.pre_s; a.pre_sumq = p.pre_sumq; a.qmax = p.qmax;
    a.gain = p.gain; a.keep = (int)p.keep;
    a.chunks = (int)(p.kp / 64);
    const bool dual = p.w1 != nullptr;
    const int64_t r = gemv_rows_per_wg(p.n, a.chunks, dual);
    a.rows_per_wg = (int)r;
    const int jm = (int)ceil_div(r * gemv_blocks(a.chunks), (int64_t)(kGT / 8));
    const dim3 grid((unsigned)ceil_div(p.n, r));
    const size_t lds = gemv_lds_bytes(p.m, p.kp, r, dual);
    if (p.pre_s) {  // quantized rows (a quantization kernel ran first)
        const int64_t sl = ceil_div(p.m * (p.kp / 16), (int64_t)kGT);
        if (sl <= 1) launch_preq<1>((int)p.m, jm, grid, lds, st, a);
        else if (sl <= 2) launch_preq<2>((int)p.m, jm, grid, lds, st, a);
        else launch_preq<4>((int)p.m, jm, grid, lds, st, a);
        return hipGetLastError();
    }
    if (p.a4) {  // one bf16 token, 4-bit codes made in the prologue (gemv_token_prologue_supported)
        const int64_t sl = ceil_div(p.k / 16, (int64_t)kGT);
        if (sl <= 1) launch_a4<1>(jm, grid, lds, st, a);
        else if (sl <= 2) launch_a4<2>(jm, grid, lds, st, a);
        else launch_a4<4>(jm, grid, lds, st, a);
        return hipGetLastError();
    }
    if (p.norm) {  // one bf16 token, normalized in the prologue (gemv_token_prologue_supported)
        const int64_t sl = ceil_div(p.k / 16, (int64_t)kGT);
        if (sl <= 1) launch_norm<1>(jm, grid, lds, st, a);
        else if (sl <= 2) launch_norm<2>(jm, grid, lds, st, a);
        else launch_norm<4>(jm, grid, lds, st, a);
        return hipGetLastError();
    }
    if (p.bf16) {
        if (dual) dispatch<bf16_t, true>(p, jm, grid, lds, st, a);
        else dispatch<bf16_t, false>(p, jm, grid, lds, st, a);
    } else {
        if (dual) dispatch<float, true>(p, jm, grid, lds, st, a);
        else dispatch<float, false>(p, jm, grid, lds, st, a);
    }
    return hipGetLastError();
}

}  // namespace bl
