// common.hpp -- device helpers shared by the gfx950 BitLinear kernels.
//
// Internal int8 activation layout ("qperm"): every token row is padded with
// zeros to kp = roundup(k, 64) bytes, and inside each 16-byte group the 4x4
// byte block is transposed: byte 4*i + b of group g holds q[16*g + 4*b + i].
// With that order, dword i of a group lines up byte-for-byte with the i-th
// 2-bit field of the packed weight dword covering the same 16 inputs
// ((w >> 2i) & 0x03030303 holds the codes of inputs 16g + 4b + i), so
// both the v_dot4 decode path and the MFMA operands read the activations
// with plain 16-byte loads and no per-element shuffles.
//
// Codes are kept as w+1 in {0,1,2}; the products then carry an offset that is
// removed once per token: sum_k q*w = sum_k q*code - sum_k q ("sumq").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: data read once, keep it out of the caches)
__device__ inline uint4 load_nt16(const void *p)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kThreads = 256;
constexpr float kEps = 1e-5f;

__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// byte offset, inside a row of the qperm layout, of input index k
__device__ inline int qperm_index(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }

// ---------------------------------------------------------------- DPP reductions
// Butterfly inside each 16-lane row with DPP (quad_perm xor1, quad_perm xor2,
// row_half_mirror, row_mirror), then across the four rows with DPP row
// broadcasts.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL>
__device__ inline int dpp_mov(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }

// Across the four rows: row_bcast:15 adds lane 15 of rows 0 and 2 into rows
// 1 and 3, row_bcast:31 lane 31 into rows 2 and 3, so lane 63 ends with the
// whole wave's result, which v_readlane hands to every lane (no LDS permute).
// Rows outside a step's row mask take `old`: v for max, 0 for sums.
__device__ inline float wave_max(float v)
{
    v = fmaxf(v, __int_as_float(dpp_mov<kDppQuadXor1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppQuadXor2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppRowHalfMirror>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppRowMirror>(__float_as_int(v))));
    int b = __float_as_int(v);
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(b, b, kDppRowBcast15, 0xA, 0xF, false)));
    b = __float_as_int(v);
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(b, b, kDppRowBcast31, 0xC, 0xF, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// maximum / sum over each row of 16 lanes (every lane of the row gets it)
__device__ inline float row16_max(float v)
{
    v = fmaxf(v, __int_as_float(dpp_mov<kDppQuadXor1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppQuadXor2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppRowHalfMirror>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_mov<kDppRowMirror>(__float_as_int(v))));
    return v;
}
__device__ inline int row16_sum(int v)
{
    v += dpp_mov<kDppQuadXor1>(v);
    v += dpp_mov<kDppQuadXor2>(v);
    v += dpp_mov<kDppRowHalfMirror>(v);
    v += dpp_mov<kDppRowMirror>(v);
    return v;
}

// sum over each group of 8 lanes (8i .. 8i+7); every lane of the group gets it
__device__ inline int group8_sum(int v)
{
    v += dpp_mov<kDppQuadXor1>(v);
    v += dpp_mov<kDppQuadXor2>(v);
    v += dpp_mov<kDppRowHalfMirror>(v);
    return v;
}

__device__ inline int wave_sum(int v)
{
    v += dpp_mov<kDppQuadXor1>(v);
    v += dpp_mov<kDppQuadXor2>(v);
    v += dpp_mov<kDppRowHalfMirror>(v);
    v += dpp_mov<kDppRowMirror>(v);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
    return __builtin_amdgcn_readlane(v, 63);
}

// ---------------------------------------------------------------- dynamic LDS limit (host)
// A launch with more dynamic LDS than the default limit needs the function's
// limit raised (hipFuncSetAttribute, per function and device). Each launching
// template instance keeps one LdsLimit; the attribute call happens only when a
// device first needs more than it was given, not on every launch.
struct LdsLimit {
    static constexpr int kDevices = 64;
    std::atomic<int> bytes[kDevices] = {};
    std::mutex mu;
};
inline hipError_t allow_dynamic_lds(const void *kern, int bytes, LdsLimit &lim)
{
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev)) return e;
    if (dev < 0 || dev >= LdsLimit::kDevices)
        return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (lim.bytes[dev].load(std::memory_order_acquire) >= bytes) return hipSuccess;
    std::lock_guard<std::mutex> g(lim.mu);
    const int have = lim.bytes[dev].load(std::memory_order_relaxed);
    if (have >= bytes) return hipSuccess;
    if (hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) return e;
    lim.bytes[dev].store(bytes, std::memory_order_release);
    return hipSuccess;
}

// ---------------------------------------------------------------- direct loads into LDS
// Direct loads from global memory into LDS with a scalar base address and a
// per-lane 32-bit byte offset. Lane i of the wave writes LDS byte address
// lds + 16*i (lds + 4*i for the dword form); lds must be wave-uniform. Issued
// as inline asm so that the only waits on these loads are the explicit ones in
// ring_barrier(): the compiler would otherwise drain every in-flight direct
// load before any LDS read. No VGPR is written by them.
// a wave-uniform 64-bit address as a scalar operand
__device__ inline uint64_t uniform_ptr(const void *p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ inline void dma16(const void *sbase, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(uniform_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
__device__ inline void dma4(const void *sbase, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(uniform_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

// LDS byte address of a pointer into the workgroup's LDS
__device__ inline uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// s_waitcnt immediate: vmcnt <= VM, lgkmcnt <= LG, expcnt untouched (gfx9 encoding)
template <int VM, int LG>
constexpr int waitcnt_vm_lgkm() { return (VM & 15) | (7 << 4) | (LG << 8) | ((VM >> 4) << 14); }

// Barrier that leaves the newest VM direct loads and the newest LG LDS reads
// in flight: wait until at most VM vector-memory and LG LDS operations of this
// thread are outstanding (both complete in issue order), then s_barrier. The
// empty asm statements keep the compiler from moving memory accesses across.
template <int VM, int LG = 0>
__device__ inline void ring_barrier()
{
    static_assert(VM < 64 && LG < 16, "waitcnt fields");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm<VM, LG>());
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- activation loads
struct bf16_t { uint16_t bits; };

__device__ inline float to_f32(float v) { return v; }
__device__ inline float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v.bits << 16); }

// Loads the 16 inputs of group g (inputs 16g .. 16g+15) of one row into f[].
// FULL: k % 16 == 0, so every group is whole and the row start is 16-byte
// aligned: straight 16-byte loads with no bounds checks (and no branches).
// Otherwise whole groups use 16-byte (fp32) or 8-byte (bf16) loads -- rows are
// at least 8-byte aligned since k % 4 == 0 -- and inputs at or beyond k read as 0.
template <typename T, bool FULL>
__device__ inline void load_group(const T *row, int64_t k, int64_t g, float f[16])
{
    const int64_t k0 = g * 16;
    if constexpr (FULL) {
        if constexpr (sizeof(T) == 4) {
            const float4 *p = reinterpret_cast<const float4 *>(row + k0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 v = p[j];
                f[4 * j + 0] = v.x; f[4 * j + 1] = v.y; f[4 * j + 2] = v.z; f[4 * j + 3] = v.w;
            }
        } else {
            const uint4 *p = reinterpret_cast<const uint4 *>(row + k0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint4 v = p[j];
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[8 * j + 2 * e + 0] = __uint_as_float(w[e] << 16);
                    f[8 * j + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            }
        }
    } else if (k0 + 16 <= k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (sizeof(T) == 4) {
                const float4 v = reinterpret_cast<const float4 *>(row + k0)[j];
                f[4 * j + 0] = v.x; f[4 * j + 1] = v.y; f[4 * j + 2] = v.z; f[4 * j + 3] = v.w;
            } else {
                const uint2 v = reinterpret_cast<const uint2 *>(row + k0)[j];
                f[4 * j + 0] = __uint_as_float(v.x << 16);
                f[4 * j + 1] = __uint_as_float(v.x & 0xFFFF0000u);
                f[4 * j + 2] = __uint_as_float(v.y << 16);
                f[4 * j + 3] = __uint_as_float(v.y & 0xFFFF0000u);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) f[j] = (k0 + j < k) ? to_f32(row[k0 + j]) : 0.0f;
    }
}

// ---------------------------------------------------------------- 4-bit activations (E2M1, top-K)
// The nearest E2M1 value of v (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives),
// doubled; at a midpoint the value with mantissa bit 0 (0, 1, 2, 4) wins.
// The E2M1 values step by 0.5 below 2, by 1 below 4 and by 2 above, so the
// doubled code is rint(|v| * 2 / d) * d with d = 1, 2, 4 in those ranges
// (|v| times a power of two is exact, and rint's ties to even are exactly the
// midpoint rule), capped at 12: no branches, and NaN gives 12.
__device__ inline int e2m1_doubled(float v)
{
    const float a = fabsf(v);
    const float up = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
    const float d = a < 2.0f ? 1.0f : (a < 4.0f ? 2.0f : 4.0f);
    const int c = (int)fminf(rintf(a * up) * d, 12.0f);
    return v < 0.0f ? -c : c;
}

// inclusive prefix sum over the 64 lanes: Kogge-Stone steps of 1, 2, 4 and 8
// inside each 16-lane row (row_shr, lanes with no source add 0), then the row
// broadcasts carry each row's total into the rows above it
__device__ inline int wave_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
    return v;
}

constexpr int kDigitBits = 11;
constexpr int kDigitBins = 1 << kDigitBits;

// The digit of the want-th largest candidate, from a histogram h of
// kDigitBins bins (bins past the digit's range hold 0); want becomes the rank
// of tau among the candidates that share that digit. Every wave computes it
// alone, with no barrier: lane L sums bins 32L .. 32L+31 (read in a rotated
// order to spread the LDS banks), a prefix sum over the lanes gives each lane
// the count above its range and so the lane whose range holds the want-th
// largest, and a second prefix sum over that lane's 32 bins gives the bin.
__device__ inline uint32_t pick_digit(const int *h, int &want)
{
    const int lane = threadIdx.x & 63;
    const int4 *hp = reinterpret_cast<const int4 *>(h + 32 * lane);
    int sl = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int4 c = hp[(i + lane) & 7];
        sl += c.x + c.y + c.z + c.w;
    }
    const int pl = wave_scan(sl);
    const int above = __builtin_amdgcn_readlane(pl, 63) - pl;  // candidates in the lanes above
    const uint64_t b1 = __ballot(above < want && want <= above + sl);
    const int ls = b1 ? __builtin_ctzll(b1) : 0;
    const int base = __builtin_amdgcn_readlane(above, ls);
    const int c = lane < 32 ? h[32 * ls + lane] : 0;
    const int p2 = wave_scan(c);
    const int ge = base + __builtin_amdgcn_readlane(p2, 31) - p2 + c;  // candidates with digit >= 32 ls + lane
    const uint64_t b2 = __ballot(lane < 32 && ge >= want && ge - c < want);
    const int lj = b2 ? __builtin_ctzll(b2) : 0;
    want -= __builtin_amdgcn_readlane(ge - c, lj);
    return (uint32_t)(32 * ls + lj);
}

// ---------------------------------------------------------------- RMS norm (subln)
// a + b = s + e exactly (Knuth's TwoSum)
__device__ inline void two_sum(double a, double b, double &s, double &e)
{
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// double-double accumulation of one value
__device__ inline void dd_add(double &hi, double &lo, double v)
{
    double e;
    two_sum(hi, v, hi, e);
    lo += e;
}

// double-double sum over a workgroup of NW waves (xor butterfly in each wave,
// then the wave results in order through LDS, red[2 * NW]); every thread gets
// the fp64 result
template <int NW>
__device__ inline double block_sum_dd(double hi, double lo, double *red)
{
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) {
        const double ph = __shfl_xor(hi, mask, 64);
        const double pl = __shfl_xor(lo, mask, 64);
        double e;
        two_sum(hi, ph, hi, e);
        lo = lo + pl + e;
    }
    if ((threadIdx.x & 63) == 0) {
        red[2 * (threadIdx.x >> 6)] = hi;
        red[2 * (threadIdx.x >> 6) + 1] = lo;
    }
    __syncthreads();
    double h = red[0], l = red[1];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        double e;
        two_sum(h, red[2 * w], h, e);
        l = l + red[2 * w + 1] + e;
    }
    return h + l;
}

// the per-token factor r = 1 / sqrt(fp32(S / k) + 1e-5)
__device__ inline float norm_factor(double ssq, int64_t k)
{
    const float ms = (float)(ssq / (double)k);
    const float d = ms + kEps;
    return 1.0f / sqrtf(d);
}

// Per-token int8 code q = clamp(rint(v * inv), -127, 127), with inv = 127 / s and
// s >= max|v|. Since |v * inv| <= 127 * (1 + 2^-23) after rounding, rint never
// leaves [-127, 127] and the clamp cannot bind. The rounding is done by adding
// 1.5 * 2^23: the sum has a unit ulp, so the add itself rounds to the nearest
// integer with ties to even (exactly rint), and the low byte of the float's bits
// is then the two's-complement int8 code. The multiply and the add are two
// separately rounded operations (no FMA contraction in this build).
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

__device__ inline uint32_t quant_bits(float v, float inv) { return __float_as_uint(v * inv + kRoundMagic); }

__device__ inline int quant_i8(float v, float inv) { return (int)(int8_t)(quant_bits(v, inv) & 0xFFu); }

// Low bytes of four quant_bits() results -> one dword (a in byte 0 ... d in byte 3).
__device__ inline uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // bytes: a0, b0, 0, 0
    const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000c0cu);  // bytes: 0, 0, c0, d0
    return lo | hi;
}

// Quantizes the 16 inputs of one group; writes the qperm order (4x4 byte
// transpose: dword i = codes of inputs i, 4+i, 8+i, 12+i) and/or the natural
// order, and returns the sum of the 16 codes.
__device__ inline int quant_group(const float f[16], float inv, uint4 *perm_out, uint4 *nat_out)
{
    uint32_t b[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) b[j] = quant_bits(f[j], inv);
    uint32_t pd[4], nd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pd[i] = pack_low_bytes(b[i], b[4 + i], b[8 + i], b[12 + i]);
        nd[i] = pack_low_bytes(b[4 * i], b[4 * i + 1], b[4 * i + 2], b[4 * i + 3]);
    }
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) sum = __builtin_amdgcn_sdot4((int)pd[i], 0x01010101, sum, false);
    if (perm_out) *perm_out = make_uint4(pd[0], pd[1], pd[2], pd[3]);
    if (nat_out) *nat_out = make_uint4(nd[0], nd[1], nd[2], nd[3]);
    return sum;
}

// The four 2-bit fields of a packed dword as int8 operand bytes: dword i holds
// (w >> 2i) & 0x03030303, the codes of inputs 16g + 4b + i for bytes b = 0..3
// of the dword covering group g -- the qperm byte order of the activations.
__device__ inline v4i expand_codes4(uint32_t w)
{
    return v4i{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
               (int)((w >> 6) & 0x03030303u)};
}

// The 16 inputs of one group from its raw 16-byte words (bf16: 2, fp32: 4),
// loaded earlier so that the conversion does not hold up other requests.
template <typename T>
__device__ inline void unpack_group(const uint4 *v, float f[16])
{
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[4 * j + 0] = __uint_as_float(v[j].x);
            f[4 * j + 1] = __uint_as_float(v[j].y);
            f[4 * j + 2] = __uint_as_float(v[j].z);
            f[4 * j + 3] = __uint_as_float(v[j].w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[8 * j + 2 * e + 0] = __uint_as_float(w[e] << 16);
                f[8 * j + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
        }
    }
}

// Packs 16 codes into the qperm byte order (used where codes are already ints).
__device__ inline uint4 qperm_pack(const int q[16])
{
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        d[i] = (uint32_t)(q[i] & 0xFF) | ((uint32_t)(q[4 + i] & 0xFF) << 8) |
               ((uint32_t)(q[8 + i] & 0xFF) << 16) | ((uint32_t)(q[12 + i] & 0xFF) << 24);
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// Rescale of one accumulator: y = (float)acc * ((s / 127) * gamma); qmax is the
// code of the largest magnitude (127 for int8 activations, 12 for the doubled
// E2M1 codes of 4-bit activations)
__device__ inline float token_scale(float s, float gamma) { return (s / 127.0f) * gamma; }
__device__ inline float token_scale(float s, float gamma, float qmax) { return (s / qmax) * gamma; }

__device__ inline float sq_relu_gate(float g, float u)
{
    float gp = g > 0.0f ? g : 0.0f;
    return (gp * gp) * u;
}

}  // namespace bl
