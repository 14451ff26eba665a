// sparse_down.hip -- the decode FFN's down projection over input-major weights,
// skipping the zero channels of the requantized h (gfx950).
//
// The FFN's gating leaves h = relu(g)^2 * u zero wherever g <= 0, and the int8
// requantization of h rounds many more of its channels to 0; only the non-zero
// channels need their weights ("BitNet 1-bit LLM 的混合精度微调技术", the
// operational-parameter paragraph: with GLU gating only the non-zero channels
// are computed). In the output-major packing [hidden][ffn/4] those zeros fall at
// scattered bytes of every row, so nothing can be skipped; in the input-major
// packing [ffn][hidden/4] (one row per channel of h) a zero channel skips a whole
// row, and the bytes read fall with the zero fraction.
//
// One launch, m <= 4 tokens. Workgroup (ks, ns) owns channel slice ks of h and
// output slice ns (512 outputs: one 128-byte line of every weight row):
//  1. s_t = max over the gate/up launch's per-workgroup maxima of |h| (then the
//     epsilon floor), inv_t = 127 / s_t: the same scale as the quantization of
//     the whole row of h;
//  2. the slice of h is quantized (the same rounding as everywhere: one fp32
//     multiply, ties to even) into LDS, and the channels where any token's
//     code is non-zero are listed (LDS atomic counter: list order does not
//     matter, the sums below are exact integers);
//  3. 8 lane groups of 32 lanes take the listed rows in turn, each lane with up
//     to 32 rows in flight; a lane reads the 4-byte word of its 16 outputs and
//     adds q * code for each, in int32;
//  4. the 8 groups' sums meet in LDS; each output's slice sum minus the slice's
//     sum of codes (the codes are w+1) is stored as this slice's int32 partial;
//  5. a second launch adds the partials of every output (integers: exact, in
//     any order) and writes y = (float)acc * ((s / 127) * gamma).
// Two launches rather than one with device-scope atomics and a last-workgroup
// rescale: on this part a device-scope release fence writes the XCD's L2 back,
// and 256 of them plus 131 K atomics cost more than the second launch
// (measured: 35 against 16.6 us for the whole 8B FFN at one token).
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kSdThreads = 256;
constexpr int kSdOut = 512;       // outputs per workgroup slice (128 bytes of a weight row)
constexpr int kSdLanes = kSdOut / 16;           // lanes per row: 4 bytes (16 outputs) each
constexpr int kSdGroups = kSdThreads / kSdLanes;  // lane groups: rows processed side by side
constexpr int kSdRows = 32;       // rows in flight per lane
constexpr int kSdMaxSlice = 1024; // channels per workgroup slice
constexpr int kSdWorkgroups = 256;

struct SparseArgs {
    const float *h;
    const float *hmax_part;
    int64_t parts;
    int64_t ffn, hidden;
    const uint8_t *wt;
    int64_t ldt;  // bytes per input-major row: hidden / 4
    int32_t *partial;  // [ks_count][MT][hidden]
    float *s;          // [MT]: the row scales, for the second launch
    int8_t *q_out;
    float *s_out;
    int ks_count, ns_count, slice;
};

template <int MT>
__global__ __launch_bounds__(kSdThreads) void sparse_down_kernel(SparseArgs a)
{
    __shared__ int q_lds[MT][kSdMaxSlice];
    __shared__ int list[kSdMaxSlice];
    __shared__ int red[kSdGroups][MT][kSdOut];
    __shared__ float red_f[MT][kSdThreads / 64];
    __shared__ int red_i[MT][kSdThreads / 64];
    __shared__ int count;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ns = blockIdx.x % a.ns_count, ks = blockIdx.x / a.ns_count;
    const int64_t k0 = (int64_t)ks * a.slice;
    const int nk = (int)((a.ffn - k0) < a.slice ? (a.ffn - k0) : a.slice);
    if (tid == 0) count = 0;

    // 1-2. this slice of h and the partial maxima of |h| are requested together
    //      (one round trip), then s_t and inv_t, then the codes of the slice go to
    //      LDS and the channels where any token's code is non-zero are listed
    constexpr int HS = kSdMaxSlice / kSdThreads;  // slice entries per thread
    float hv[MT][HS];
#pragma unroll
    for (int r = 0; r < HS; ++r) {
        const int i = tid + r * kSdThreads;
#pragma unroll
        for (int t = 0; t < MT; ++t) hv[t][r] = i < nk ? a.h[t * a.ffn + k0 + i] : 0.0f;
    }
    float st[MT], inv[MT];
    {
        float mx[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) mx[t] = 0.0f;
        for (int64_t i = tid; i < a.parts; i += kSdThreads)
#pragma unroll
            for (int t = 0; t < MT; ++t) mx[t] = fmaxf(mx[t], a.hmax_part[i * MT + t]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            mx[t] = wave_max(mx[t]);
            if (lane == 0) red_f[t][wave] = mx[t];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float m = red_f[t][0];
#pragma unroll
            for (int w = 1; w < kSdThreads / 64; ++w) m = fmaxf(m, red_f[t][w]);
            st[t] = fmaxf(m, kEps);
            inv[t] = 127.0f / st[t];
        }
    }
    int qsum[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) qsum[t] = 0;
#pragma unroll
    for (int r = 0; r < HS; ++r) {
        const int i = tid + r * kSdThreads;
        if (i < nk) {
            bool nz = false;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int q = quant_i8(hv[t][r], inv[t]);
                q_lds[t][i] = q;
                qsum[t] += q;
                nz |= q != 0;
                if (a.q_out && ns == 0) a.q_out[t * a.ffn + k0 + i] = (int8_t)q;
            }
            if (nz) list[atomicAdd(&count, 1)] = i;
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int sw = wave_sum(qsum[t]);
        if (lane == 0) red_i[t][wave] = sw;
    }
    if (blockIdx.x == 0 && tid < MT) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
            if (t == tid) {
                a.s[t] = st[t];
                if (a.s_out) a.s_out[t] = st[t];
            }
    }
    __syncthreads();
    const int cnt = count;

    // 3. the listed rows: groups of 32 lanes, a lane's word holds 16 outputs
    const int grp = tid / kSdLanes, li = tid % kSdLanes;
    const int64_t out0 = (int64_t)ns * kSdOut + 16 * li;  // first output of this lane's word
    const bool live = out0 < a.hidden;
    const uint8_t *col = a.wt + (int64_t)ns * (kSdOut / 4) + 4 * li;
    int acc[MT][16];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[t][j] = 0;
    constexpr int U = kSdRows;
    for (int i0 = grp; i0 < cnt; i0 += kSdGroups * U) {
        uint32_t w[U];
        int kk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kSdGroups;
            kk[u] = i < cnt ? list[i] : -1;
            w[u] = (kk[u] >= 0 && live) ? *reinterpret_cast<const uint32_t *>(col + (k0 + kk[u]) * a.ldt) : 0x55555555u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kk[u] < 0) continue;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int q = q_lds[t][kk[u]];
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[t][j] += q * (int)((w[u] >> (2 * j)) & 3u);
            }
        }
    }

    // 4. the groups' sums meet in LDS; one partial per output and token
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) red[grp][t][16 * li + j] = acc[t][j];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int slice_sum = red_i[t][0] + red_i[t][1] + red_i[t][2] + red_i[t][3];
#pragma unroll
        for (int o = tid; o < kSdOut; o += kSdThreads) {
            const int64_t n = (int64_t)ns * kSdOut + o;
            int v = 0;
#pragma unroll
            for (int g = 0; g < kSdGroups; ++g) v += red[g][t][o];
            if (n < a.hidden) a.partial[((int64_t)ks * MT + t) * a.hidden + n] = v - slice_sum;
        }
    }
}

// y = (float)(sum of the slices' partials) * ((s / 127) * gamma). A workgroup
// takes 64 outputs; its four waves each add every fourth slice, eight loads in
// flight per lane, and meet in LDS.
template <int MT>
__global__ __launch_bounds__(256) void sparse_down_finish_kernel(const int32_t *__restrict__ partial, int ks_count,
                                                                 int64_t hidden, const float *__restrict__ s,
                                                                 const float *__restrict__ gamma, float *__restrict__ y)
{
    __shared__ int red[4][MT][64];
    const int o = threadIdx.x & 63, ph = threadIdx.x >> 6;
    const int64_t n = (int64_t)blockIdx.x * 64 + o;
    const bool live = n < hidden;
    int v[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) v[t] = 0;
    for (int k0 = ph; k0 < ks_count; k0 += 32) {
        int p[MT][8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = k0 + 4 * j;
#pragma unroll
            for (int t = 0; t < MT; ++t)
                p[t][j] = (live && k < ks_count) ? partial[((int64_t)k * MT + t) * hidden + n] : 0;
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int j = 0; j < 8; ++j) v[t] += p[t][j];
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) red[ph][t][o] = v[t];
    __syncthreads();
    if (ph == 0 && live) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int acc = red[0][t][o] + red[1][t][o] + red[2][t][o] + red[3][t][o];
            y[t * hidden + n] = (float)acc * token_scale(s[t], gamma[0]);
        }
    }
}

int64_t sparse_down_nslices(int64_t hidden) { return ceil_div(hidden, (int64_t)kSdOut); }

static int sparse_down_kslices(int64_t hidden, int64_t ffn)
{
    const int64_t ns = sparse_down_nslices(hidden);
    int64_t ks = ceil_div((int64_t)kSdWorkgroups, ns);
    if (ks < 1) ks = 1;
    if (ceil_div(ffn, ks) > kSdMaxSlice) ks = ceil_div(ffn, (int64_t)kSdMaxSlice);
    if (ks > ffn) ks = ffn;
    return (int)ks;
}

int64_t sparse_down_partials(int64_t hidden, int64_t ffn) { return sparse_down_kslices(hidden, ffn); }

template <int MT>
static void launch_mt(const SparseArgs &a, const float *gamma, float *y, hipStream_t st)
{
    hipLaunchKernelGGL(sparse_down_kernel<MT>, dim3((unsigned)(a.ks_count * a.ns_count)), dim3(kSdThreads), 0, st,
                       a);
    hipLaunchKernelGGL(sparse_down_finish_kernel<MT>, dim3((unsigned)ceil_div(a.hidden, (int64_t)64)), dim3(256),
                       0, st, a.partial, a.ks_count, a.hidden, a.s, gamma, y);
}

hipError_t launch_sparse_down(const SparseDownProblem &p, hipStream_t st)
{
    SparseArgs a;
    a.h = p.h; a.hmax_part = p.hmax_part; a.parts = p.parts;
    a.ffn = p.ffn; a.hidden = p.hidden; a.wt = p.wt; a.ldt = p.hidden / 4;
    a.partial = p.partial; a.s = p.s;
    a.q_out = p.q_out; a.s_out = p.s_out;
    a.ns_count = (int)sparse_down_nslices(p.hidden);
    a.ks_count = sparse_down_kslices(p.hidden, p.ffn);
    a.slice = (int)ceil_div(p.ffn, (int64_t)a.ks_count);
    switch (p.m) {
    case 1: launch_mt<1>(a, p.gamma, p.y, st); break;
    case 2: launch_mt<2>(a, p.gamma, p.y, st); break;
    case 3: launch_mt<3>(a, p.gamma, p.y, st); break;
    default: launch_mt<4>(a, p.gamma, p.y, st); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- input-major packing
// One output byte per thread: the codes of outputs 4j..4j+3 at input c.
__global__ __launch_bounds__(256) void pack_kmajor_kernel(const uint8_t *__restrict__ packed, int64_t n, int64_t k,
                                                          uint8_t *__restrict__ out)
{
    const int64_t nb = n / 4, kb = k / 4;
    const int64_t total = k * nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = i / nb, j = i - c * nb;
        const int sh = 2 * (int)(c & 3);
        uint32_t byte = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) byte |= (uint32_t)((packed[(4 * j + r) * kb + (c >> 2)] >> sh) & 3) << (2 * r);
        out[i] = (uint8_t)byte;
    }
}

hipError_t launch_pack_kmajor(const uint8_t *packed, int64_t n, int64_t k, uint8_t *packed_t, hipStream_t st)
{
    const int64_t total = k * (n / 4);
    int64_t blocks = ceil_div(total, 256);
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(pack_kmajor_kernel, dim3((unsigned)blocks), dim3(256), 0, st, packed, n, k, packed_t);
    return hipGetLastError();
}

}  // namespace bl
