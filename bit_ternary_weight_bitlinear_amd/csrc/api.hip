// api.hip -- the extern "C" boundary of the gfx950 BitLinear library.
//
// Every entry point validates its arguments on the host before anything is
// enqueued, lays out the caller's workspace, and enqueues kernels on the
// caller's stream. Nothing here allocates, synchronises or keeps state.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "../../include/bitlinear.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace bl;

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kRowPad = 256;  // activation rows are padded to the largest GEMM row tile

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void *p) { return aligned(p, 16); }

bool dim_ok(int64_t d) { return d >= 1 && d <= BL_MAX_DIM; }
bool kdim_ok(int64_t k) { return k >= 4 && k <= BL_MAX_DIM && k % 4 == 0; }
bool tokens_ok(int64_t m) { return m >= 1 && m <= BL_MAX_TOKENS; }

// bump allocator over the caller's workspace
struct Carve {
    char *base;
    int64_t off = 0;
    explicit Carve(void *b) : base(static_cast<char *>(b)) {}
    template <typename T>
    T *take(int64_t bytes)
    {
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += round_up(bytes, kAlign);
        return p;
    }
};

// ---- layouts (shared by the size query and the calls)
struct FwdLayout {
    bool gemv;
    int64_t kp;
    int8_t *qp = nullptr;
    float *s = nullptr;
    int32_t *sumq = nullptr;
    uint8_t *wpad = nullptr;
    int64_t bytes = 0;
};

// force_gemm: the activations always go through the quantization kernel into
// the workspace (the bare integer product, and the normalized forward)
FwdLayout forward_layout(void *ws, int64_t m, int64_t k, int64_t n, bool force_gemm)
{
    FwdLayout L;
    L.kp = round_up(k, 64);
    L.gemv = !force_gemm && gemv_supported(m, L.kp);
    Carve c(ws);
    if (!L.gemv) {
        const int64_t mp = round_up(m, kRowPad);
        L.qp = c.take<int8_t>(mp * L.kp);
        L.s = c.take<float>(mp * 4);
        L.sumq = c.take<int32_t>(mp * 4);
    }
    if (k % 64) L.wpad = c.take<uint8_t>(n * (L.kp / 4));
    L.bytes = c.off;
    return L;
}

struct FfnLayout {
    bool gemv;
    int64_t hp, fp;
    int8_t *qx = nullptr, *qh = nullptr;
    float *sx = nullptr, *sh = nullptr, *h = nullptr;
    int32_t *sumx = nullptr, *sumh = nullptr;
    uint8_t *gpad = nullptr, *upad = nullptr, *dpad = nullptr;
    int64_t bytes = 0;
};

FfnLayout ffn_layout(void *ws, int64_t m, int64_t hidden, int64_t ffn)
{
    FfnLayout L;
    L.hp = round_up(hidden, 64);
    L.fp = round_up(ffn, 64);
    L.gemv = gemv_supported(m, L.hp) && gemv_supported(m, L.fp);
    Carve c(ws);
    L.h = c.take<float>(m * ffn * 4);
    if (!L.gemv) {
        const int64_t mp = round_up(m, kRowPad);
        L.qx = c.take<int8_t>(mp * L.hp);
        L.sx = c.take<float>(mp * 4);
        L.sumx = c.take<int32_t>(mp * 4);
        L.qh = c.take<int8_t>(mp * L.fp);
        L.sh = c.take<float>(mp * 4);
        L.sumh = c.take<int32_t>(mp * 4);
    }
    if (hidden % 64) {
        L.gpad = c.take<uint8_t>(ffn * (L.hp / 4));
        L.upad = c.take<uint8_t>(ffn * (L.hp / 4));
    }
    if (ffn % 64) L.dpad = c.take<uint8_t>(hidden * (L.fp / 4));
    L.bytes = c.off;
    return L;
}

struct SparseFfnLayout {
    int64_t hp;
    int64_t parts;
    float *h = nullptr, *hmax = nullptr, *s = nullptr;
    int32_t *partial = nullptr;  // [slices of ffn][m][hidden]
    uint8_t *gpad = nullptr, *upad = nullptr;
    int64_t bytes = 0;
};

SparseFfnLayout sparse_ffn_layout(void *ws, int64_t m, int64_t hidden, int64_t ffn)
{
    SparseFfnLayout L;
    L.hp = round_up(hidden, 64);
    L.parts = gemv_grid(ffn, L.hp, true);
    Carve c(ws);
    L.h = c.take<float>(m * ffn * 4);
    L.hmax = c.take<float>(L.parts * m * 4);
    L.s = c.take<float>(m * 4);
    L.partial = c.take<int32_t>(sparse_down_partials(hidden, ffn) * m * hidden * 4);
    if (hidden % 64) {
        L.gpad = c.take<uint8_t>(ffn * (L.hp / 4));
        L.upad = c.take<uint8_t>(ffn * (L.hp / 4));
    }
    L.bytes = c.off;
    return L;
}

bool sparse_ffn_shape_ok(int64_t m, int64_t hidden, int64_t ffn)
{
    return m >= 1 && m <= 4 && kdim_ok(hidden) && hidden % 16 == 0 && kdim_ok(ffn) &&
           gemv_supported(m, round_up(hidden, 64));
}

bl_status hip_status(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

// argument checks of the forward (shared by bitlinear_forward and its variant
// without a workspace argument)
bl_status forward_args(const void *x, bl_dtype dtype, int64_t m, int64_t k, const uint8_t *packed,
                       const float *gamma, int64_t n, const float *y, const int32_t *acc_out)
{
    if (!x || !packed || !gamma || !y) return BL_ERR_NULL;
    if (dtype != BL_F32 && dtype != BL_BF16) return BL_ERR_DTYPE;
    if (!tokens_ok(m) || !kdim_ok(k) || !dim_ok(n)) return BL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(y) || !aligned(gamma, 4) ||
        (acc_out && !aligned16(acc_out)))
        return BL_ERR_ALIGN;
    return BL_OK;
}

// ---- the library-owned scratch of bitlinear_forward_noalloc
// One array per device, in the code object's zero-initialised data (no file
// space), held by every device the library runs on until the process ends.
// Its device address is looked up once per device and cached; host code never
// passes the symbol itself to a kernel (on the host it is only a stand-in).
static __device__ __align__(256) uint8_t scratch[BL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

bl_status scratch_address(hipStream_t st, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BL_ERR_HIP;
    if (st) {
        int sdev = -1;
        if (hipStreamGetDevice(st, &sdev) != hipSuccess) return BL_ERR_HIP;
        if (sdev != dev) return BL_ERR_VALUE;  // the stream must belong to the current device
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BL_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BL_OK;
}

bl_status check_ws(void *ws, size_t ws_bytes, int64_t need)
{
    if (need == 0) return BL_OK;
    if (!ws) return BL_ERR_NULL;
    if (!aligned(ws, kAlign)) return BL_ERR_ALIGN;
    if ((int64_t)ws_bytes < need) return BL_ERR_WORKSPACE;
    return BL_OK;
}

}  // namespace

extern "C" {

size_t bitlinear_workspace_size(int op, int64_t m, int64_t k, int64_t n)
{
    switch (op) {
    case BL_OP_PACK:
        if (!dim_ok(n) || !kdim_ok(k)) return 0;
        return (size_t)round_up(n * 8, kAlign);
    case BL_OP_FORWARD:
        if (!tokens_ok(m) || !kdim_ok(k) || !dim_ok(n)) return 0;
        return (size_t)forward_layout(nullptr, m, k, n, false).bytes;
    case BL_OP_GEMM_I32:
        if (!tokens_ok(m) || !kdim_ok(k) || !dim_ok(n)) return 0;
        return (size_t)forward_layout(nullptr, m, k, n, true).bytes;
    case BL_OP_FFN:
        if (!tokens_ok(m) || !kdim_ok(k) || !kdim_ok(n)) return 0;
        return (size_t)ffn_layout(nullptr, m, k, n).bytes;
    case BL_OP_PACK_THRESHOLD:
        if (!dim_ok(n) || !kdim_ok(k)) return 0;
        return (size_t)(round_up(n * 8, kAlign) + kAlign);
    case BL_OP_FORWARD_NORM:
        if (!tokens_ok(m) || !kdim_ok(k) || !dim_ok(n)) return 0;
        return (size_t)forward_layout(nullptr, m, k, n, true).bytes;
    case BL_OP_FORWARD_A4:
        if (!tokens_ok(m) || !kdim_ok(k) || !dim_ok(n)) return 0;
        return (size_t)forward_layout(nullptr, m, k, n, true).bytes;
    case BL_OP_FFN_SPARSE:
        if (!sparse_ffn_shape_ok(m, k, n)) return 0;
        return (size_t)sparse_ffn_layout(nullptr, m, k, n).bytes;
    default:
        return 0;
    }
}

const char *bitlinear_status_string(bl_status status)
{
    switch (status) {
    case BL_OK: return "BL_OK";
    case BL_ERR_NULL: return "BL_ERR_NULL: a required pointer is NULL";
    case BL_ERR_SHAPE: return "BL_ERR_SHAPE: invalid shape (m, n >= 1; k >= 4, k % 4 == 0; within limits)";
    case BL_ERR_ALIGN: return "BL_ERR_ALIGN: a device pointer is not suitably aligned";
    case BL_ERR_DTYPE: return "BL_ERR_DTYPE: unknown activation dtype";
    case BL_ERR_WORKSPACE: return "BL_ERR_WORKSPACE: workspace smaller than bitlinear_workspace_size()";
    case BL_ERR_HIP: return "BL_ERR_HIP: a kernel launch failed";
    case BL_ERR_VALUE: return "BL_ERR_VALUE: a scalar argument is out of range";
    default: return "unknown bitlinear status";
    }
}

bl_status bitlinear_pack_weights(const float *w, int64_t n, int64_t k, uint8_t *packed, float *gamma,
                                 void *workspace, size_t workspace_bytes, void *stream)
{
    if (!w || !packed || !gamma) return BL_ERR_NULL;
    if (!dim_ok(n) || !kdim_ok(k)) return BL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(packed) || !aligned(gamma, 4)) return BL_ERR_ALIGN;
    const bl_status ws = check_ws(workspace, workspace_bytes, round_up(n * 8, kAlign));
    if (ws != BL_OK) return ws;
    return hip_status(launch_pack(w, n, k, packed, gamma, static_cast<double *>(workspace),
                                  static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_pack_weights_threshold(const float *w, int64_t n, int64_t k, float delta_factor,
                                           uint8_t *packed, float *alpha, float *delta_out, void *workspace,
                                           size_t workspace_bytes, void *stream)
{
    if (!w || !packed || !alpha) return BL_ERR_NULL;
    if (!dim_ok(n) || !kdim_ok(k)) return BL_ERR_SHAPE;
    if (!(delta_factor >= 0.0f) || !(delta_factor <= 3.402823466e38f)) return BL_ERR_VALUE;  // NaN fails both
    if (!aligned16(w) || !aligned16(packed) || !aligned(alpha, 4) || (delta_out && !aligned(delta_out, 4)))
        return BL_ERR_ALIGN;
    const int64_t sums = round_up(n * 8, kAlign);
    const bl_status ws = check_ws(workspace, workspace_bytes, sums + kAlign);
    if (ws != BL_OK) return ws;
    float *delta = delta_out ? delta_out : reinterpret_cast<float *>(static_cast<char *>(workspace) + sums);
    return hip_status(launch_pack_threshold(w, n, k, delta_factor, packed, alpha, delta,
                                            static_cast<double *>(workspace), static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_quant_act(const void *x, bl_dtype dtype, int64_t m, int64_t k, int8_t *q, float *scale,
                              void *stream)
{
    if (!x || !q || !scale) return BL_ERR_NULL;
    if (dtype != BL_F32 && dtype != BL_BF16) return BL_ERR_DTYPE;
    if (!tokens_ok(m) || !kdim_ok(k)) return BL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned(scale, 4)) return BL_ERR_ALIGN;
    return hip_status(launch_act_quant(x, dtype == BL_BF16, m, k, round_up(k, 64), q, nullptr, scale,
                                       nullptr, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_quant_act_norm(const void *x, bl_dtype dtype, int64_t m, int64_t k, const float *gain,
                                   int8_t *q, float *scale, void *stream)
{
    if (!x || !q || !scale) return BL_ERR_NULL;
    if (dtype != BL_F32 && dtype != BL_BF16) return BL_ERR_DTYPE;
    if (!tokens_ok(m) || !kdim_ok(k)) return BL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned(scale, 4) || (gain && !aligned16(gain))) return BL_ERR_ALIGN;
    return hip_status(launch_act_quant_norm(x, dtype == BL_BF16, m, k, round_up(k, 64), gain, q, nullptr, scale,
                                            nullptr, static_cast<hipStream_t>(stream)));
}

// The contraction of activations quantized into the workspace (qperm rows,
// scales, code sums) by one of the quantization kernels; qmax as in token_scale.
bl_status prequant_contraction(const FwdLayout &L, int64_t m, int64_t k, int64_t n, const uint8_t *w,
                               const float *gamma, float *y, int32_t *acc_out, float qmax, hipStream_t st)
{
    if (gemv_prequant_supported(m, L.kp)) {  // 1..4 tokens: the decode kernel
        GemvProblem p{};
        p.x = L.qp; p.bf16 = false; p.m = m; p.k = k; p.kp = L.kp; p.n = n;
        p.w0 = w; p.ldw = L.kp / 4; p.gamma0 = gamma; p.out = y; p.acc_out = acc_out;
        p.pre_s = L.s; p.pre_sumq = L.sumq; p.qmax = qmax;
        return hip_status(launch_gemv(p, st));
    }
    GemmProblem g{};
    g.qp = L.qp; g.kp = L.kp; g.s = L.s; g.sumq = L.sumq; g.m = m; g.n = n;
    g.w0 = w; g.w1 = nullptr; g.ldw = L.kp / 4; g.gamma0 = gamma; g.gamma1 = nullptr;
    g.out = y; g.acc_out = acc_out; g.epi = EPI_Y; g.qmax = qmax;
    return hip_status(launch_contraction(g, st));
}

bl_status bitlinear_forward_norm(const void *x, bl_dtype dtype, int64_t m, int64_t k, const float *gain,
                                 const uint8_t *packed, const float *gamma, int64_t n, float *y, int32_t *acc_out,
                                 void *workspace, size_t workspace_bytes, void *stream)
{
    if (const bl_status a = forward_args(x, dtype, m, k, packed, gamma, n, y, acc_out)) return a;
    if (gain && !aligned16(gain)) return BL_ERR_ALIGN;
    const FwdLayout need = forward_layout(nullptr, m, k, n, true);
    if (const bl_status w = check_ws(workspace, workspace_bytes, need.bytes)) return w;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const FwdLayout L = forward_layout(workspace, m, k, n, true);
    const uint8_t *w = packed;
    if (L.wpad) {
        if (hipError_t e = launch_pad_weights(packed, n, k, L.kp, L.wpad, st)) return hip_status(e);
        w = L.wpad;
    }
    if (gemv_token_prologue_supported(m, k, dtype == BL_BF16)) {  // one token: the norm in the decode kernel's prologue
        GemvProblem p{};
        p.x = x; p.bf16 = true; p.m = m; p.k = k; p.kp = L.kp; p.n = n;
        p.w0 = w; p.ldw = L.kp / 4; p.gamma0 = gamma; p.out = y; p.acc_out = acc_out;
        p.norm = true; p.gain = gain;
        return hip_status(launch_gemv(p, st));
    }
    if (hipError_t e = launch_act_quant_norm(x, dtype == BL_BF16, m, k, L.kp, gain, nullptr, L.qp, L.s, L.sumq, st))
        return hip_status(e);
    return prequant_contraction(L, m, k, n, w, gamma, y, acc_out, 127.0f, st);
}

bl_status bitlinear_quant_act_a4(const void *x, bl_dtype dtype, int64_t m, int64_t k, int64_t keep, int8_t *q,
                                 float *scale, void *stream)
{
    if (!x || !q || !scale) return BL_ERR_NULL;
    if (dtype != BL_F32 && dtype != BL_BF16) return BL_ERR_DTYPE;
    if (!tokens_ok(m) || !kdim_ok(k)) return BL_ERR_SHAPE;
    if (keep < 1 || keep > k) return BL_ERR_VALUE;
    if (!aligned16(x) || !aligned16(q) || !aligned(scale, 4)) return BL_ERR_ALIGN;
    return hip_status(launch_act_quant_a4(x, dtype == BL_BF16, m, k, round_up(k, 64), keep, q, nullptr, scale,
                                          nullptr, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_forward_a4(const void *x, bl_dtype dtype, int64_t m, int64_t k, int64_t keep,
                               const uint8_t *packed, const float *gamma, int64_t n, float *y, int32_t *acc_out,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (const bl_status a = forward_args(x, dtype, m, k, packed, gamma, n, y, acc_out)) return a;
    if (keep < 1 || keep > k) return BL_ERR_VALUE;
    const FwdLayout need = forward_layout(nullptr, m, k, n, true);
    if (const bl_status w = check_ws(workspace, workspace_bytes, need.bytes)) return w;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const FwdLayout L = forward_layout(workspace, m, k, n, true);
    const uint8_t *w = packed;
    if (L.wpad) {
        if (hipError_t e = launch_pad_weights(packed, n, k, L.kp, L.wpad, st)) return hip_status(e);
        w = L.wpad;
    }
    if (gemv_token_prologue_supported(m, k, dtype == BL_BF16)) {  // one token: the 4-bit codes in the decode kernel's prologue
        GemvProblem p{};
        p.x = x; p.bf16 = true; p.m = m; p.k = k; p.kp = L.kp; p.n = n;
        p.w0 = w; p.ldw = L.kp / 4; p.gamma0 = gamma; p.out = y; p.acc_out = acc_out;
        p.a4 = true; p.keep = keep; p.qmax = 12.0f;
        return hip_status(launch_gemv(p, st));
    }
    if (hipError_t e = launch_act_quant_a4(x, dtype == BL_BF16, m, k, L.kp, keep, nullptr, L.qp, L.s, L.sumq, st))
        return hip_status(e);
    return prequant_contraction(L, m, k, n, w, gamma, y, acc_out, 12.0f, st);
}

bl_status bitlinear_forward(const void *x, bl_dtype dtype, int64_t m, int64_t k, const uint8_t *packed,
                            const float *gamma, int64_t n, float *y, int32_t *acc_out, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    if (const bl_status a = forward_args(x, dtype, m, k, packed, gamma, n, y, acc_out)) return a;
    const FwdLayout need = forward_layout(nullptr, m, k, n, false);
    const bl_status wss = check_ws(workspace, workspace_bytes, need.bytes);
    if (wss != BL_OK) return wss;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const FwdLayout L = forward_layout(workspace, m, k, n, false);
    const uint8_t *w = packed;
    if (L.wpad) {
        if (hipError_t e = launch_pad_weights(packed, n, k, L.kp, L.wpad, st)) return hip_status(e);
        w = L.wpad;
    }
    if (L.gemv) {
        GemvProblem p{};
        p.x = x; p.bf16 = dtype == BL_BF16; p.m = m; p.k = k; p.kp = L.kp; p.n = n;
        p.w0 = w; p.w1 = nullptr; p.ldw = L.kp / 4; p.gamma0 = gamma; p.gamma1 = nullptr;
        p.out = y; p.acc_out = acc_out;
        return hip_status(launch_gemv(p, st));
    }
    if (bgemv_supported(m, k, dtype == BL_BF16)) {  // 5..16 tokens: quantization, products and rescale in one launch
        GemvProblem bp{};
        bp.x = x; bp.bf16 = dtype == BL_BF16; bp.m = m; bp.k = k; bp.kp = L.kp; bp.n = n;
        bp.w0 = w; bp.ldw = L.kp / 4; bp.gamma0 = gamma;
        bp.out = y; bp.acc_out = acc_out;
        return hip_status(launch_bgemv(bp, st));
    }
    if (hipError_t e = launch_act_quant(x, dtype == BL_BF16, m, k, L.kp, nullptr, L.qp, L.s, L.sumq, st))
        return hip_status(e);
    GemmProblem g{};
    g.qp = L.qp; g.kp = L.kp; g.s = L.s; g.sumq = L.sumq; g.m = m; g.n = n;
    g.w0 = w; g.w1 = nullptr; g.ldw = L.kp / 4; g.gamma0 = gamma; g.gamma1 = nullptr;
    g.out = y; g.acc_out = acc_out; g.epi = EPI_Y;
    return hip_status(launch_contraction(g, st));
}

bl_status bitlinear_forward_noalloc(const void *x, bl_dtype dtype, int64_t m, int64_t k, const uint8_t *packed,
                                    const float *gamma, int64_t n, float *y, int32_t *acc_out, void *stream)
{
    if (const bl_status a = forward_args(x, dtype, m, k, packed, gamma, n, y, acc_out)) return a;
    const int64_t need = forward_layout(nullptr, m, k, n, false).bytes;
    if (need > BL_NOALLOC_SCRATCH_BYTES) return BL_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        if (const bl_status e = scratch_address(static_cast<hipStream_t>(stream), &ws)) return e;
    }
    return bitlinear_forward(x, dtype, m, k, packed, gamma, n, y, acc_out, ws,
                             need > 0 ? (size_t)BL_NOALLOC_SCRATCH_BYTES : 0, stream);
}

bl_status bitlinear_pack_kmajor(const uint8_t *packed, int64_t n, int64_t k, uint8_t *packed_t, void *stream)
{
    if (!packed || !packed_t) return BL_ERR_NULL;
    if (!dim_ok(n) || n % 4 || !kdim_ok(k)) return BL_ERR_SHAPE;
    if (!aligned16(packed) || !aligned16(packed_t)) return BL_ERR_ALIGN;
    return hip_status(launch_pack_kmajor(packed, n, k, packed_t, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_ffn_sparse(const void *x, bl_dtype dtype, int64_t m, int64_t hidden, int64_t ffn,
                               const uint8_t *gate_packed, const float *gate_gamma, const uint8_t *up_packed,
                               const float *up_gamma, const uint8_t *down_packed_t, const float *down_gamma,
                               float *y, int8_t *hq_out, float *hs_out, void *workspace, size_t workspace_bytes,
                               void *stream)
{
    if (!x || !gate_packed || !gate_gamma || !up_packed || !up_gamma || !down_packed_t || !down_gamma || !y)
        return BL_ERR_NULL;
    if (dtype != BL_F32 && dtype != BL_BF16) return BL_ERR_DTYPE;
    if (!sparse_ffn_shape_ok(m, hidden, ffn)) return BL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(gate_packed) || !aligned16(up_packed) || !aligned16(down_packed_t) ||
        !aligned16(y) || !aligned(gate_gamma, 4) || !aligned(up_gamma, 4) || !aligned(down_gamma, 4) ||
        (hq_out && !aligned16(hq_out)) || (hs_out && !aligned(hs_out, 4)))
        return BL_ERR_ALIGN;
    const SparseFfnLayout need = sparse_ffn_layout(nullptr, m, hidden, ffn);
    if (const bl_status w = check_ws(workspace, workspace_bytes, need.bytes)) return w;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const SparseFfnLayout L = sparse_ffn_layout(workspace, m, hidden, ffn);
    const uint8_t *wg = gate_packed, *wu = up_packed;
    if (L.gpad) {
        if (hipError_t e = launch_pad_weights(gate_packed, ffn, hidden, L.hp, L.gpad, st)) return hip_status(e);
        if (hipError_t e = launch_pad_weights(up_packed, ffn, hidden, L.hp, L.upad, st)) return hip_status(e);
        wg = L.gpad;
        wu = L.upad;
    }
    GemvProblem p{};
    p.x = x; p.bf16 = dtype == BL_BF16; p.m = m; p.k = hidden; p.kp = L.hp; p.n = ffn;
    p.w0 = wg; p.w1 = wu; p.ldw = L.hp / 4; p.gamma0 = gate_gamma; p.gamma1 = up_gamma;
    p.out = L.h; p.hmax_part = L.hmax;
    if (hipError_t e = launch_gemv(p, st)) return hip_status(e);
    SparseDownProblem d{};
    d.h = L.h; d.hmax_part = L.hmax; d.parts = L.parts; d.m = m; d.ffn = ffn; d.hidden = hidden;
    d.wt = down_packed_t; d.gamma = down_gamma; d.y = y;
    d.partial = L.partial; d.s = L.s;
    d.q_out = hq_out; d.s_out = hs_out;
    return hip_status(launch_sparse_down(d, st));
}

bl_status bitlinear_gemm_i32(const int8_t *q, int64_t m, int64_t k, const uint8_t *packed, int64_t n,
                             int32_t *acc, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !packed || !acc) return BL_ERR_NULL;
    if (!tokens_ok(m) || !kdim_ok(k) || !dim_ok(n)) return BL_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(packed) || !aligned16(acc)) return BL_ERR_ALIGN;
    const FwdLayout need = forward_layout(nullptr, m, k, n, true);
    const bl_status wss = check_ws(workspace, workspace_bytes, need.bytes);
    if (wss != BL_OK) return wss;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const FwdLayout L = forward_layout(workspace, m, k, n, true);
    const uint8_t *w = packed;
    if (L.wpad) {
        if (hipError_t e = launch_pad_weights(packed, n, k, L.kp, L.wpad, st)) return hip_status(e);
        w = L.wpad;
    }
    if (hipError_t e = launch_perm_q(q, m, k, L.kp, L.qp, L.sumq, st)) return hip_status(e);
    GemmProblem g{};
    g.qp = L.qp; g.kp = L.kp; g.s = nullptr; g.sumq = L.sumq; g.m = m; g.n = n;
    g.w0 = w; g.w1 = nullptr; g.ldw = L.kp / 4; g.gamma0 = nullptr; g.gamma1 = nullptr;
    g.out = nullptr; g.acc_out = acc; g.epi = EPI_ACC;
    return hip_status(launch_contraction(g, st));
}

bl_status bitlinear_ffn(const void *x, bl_dtype dtype, int64_t m, int64_t hidden, int64_t ffn,
                        const uint8_t *gate_packed, const float *gate_gamma, const uint8_t *up_packed,
                        const float *up_gamma, const uint8_t *down_packed, const float *down_gamma,
                        float *y, int8_t *hq_out, float *hs_out, void *workspace, size_t workspace_bytes,
                        void *stream)
{
    if (!x || !gate_packed || !gate_gamma || !up_packed || !up_gamma || !down_packed || !down_gamma || !y)
        return BL_ERR_NULL;
    if (dtype != BL_F32 && dtype != BL_BF16) return BL_ERR_DTYPE;
    if (!tokens_ok(m) || !kdim_ok(hidden) || !kdim_ok(ffn)) return BL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(gate_packed) || !aligned16(up_packed) || !aligned16(down_packed) ||
        !aligned16(y) || !aligned(gate_gamma, 4) || !aligned(up_gamma, 4) || !aligned(down_gamma, 4) ||
        (hq_out && !aligned16(hq_out)) || (hs_out && !aligned(hs_out, 4)))
        return BL_ERR_ALIGN;
    const FfnLayout need = ffn_layout(nullptr, m, hidden, ffn);
    const bl_status wss = check_ws(workspace, workspace_bytes, need.bytes);
    if (wss != BL_OK) return wss;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const FfnLayout L = ffn_layout(workspace, m, hidden, ffn);
    const uint8_t *wg = gate_packed, *wu = up_packed, *wd = down_packed;
    if (L.gpad) {
        if (hipError_t e = launch_pad_weights(gate_packed, ffn, hidden, L.hp, L.gpad, st)) return hip_status(e);
        if (hipError_t e = launch_pad_weights(up_packed, ffn, hidden, L.hp, L.upad, st)) return hip_status(e);
        wg = L.gpad;
        wu = L.upad;
    }
    if (L.dpad) {
        if (hipError_t e = launch_pad_weights(down_packed, hidden, ffn, L.fp, L.dpad, st)) return hip_status(e);
        wd = L.dpad;
    }
    if (L.gemv) {
        GemvProblem p{};
        p.x = x; p.bf16 = dtype == BL_BF16; p.m = m; p.k = hidden; p.kp = L.hp; p.n = ffn;
        p.w0 = wg; p.w1 = wu; p.ldw = L.hp / 4; p.gamma0 = gate_gamma; p.gamma1 = up_gamma;
        p.out = L.h;
        if (hipError_t e = launch_gemv(p, st)) return hip_status(e);
        GemvProblem d{};
        d.x = L.h; d.bf16 = false; d.m = m; d.k = ffn; d.kp = L.fp; d.n = hidden;
        d.w0 = wd; d.w1 = nullptr; d.ldw = L.fp / 4; d.gamma0 = down_gamma; d.gamma1 = nullptr;
        d.out = y; d.acc_out = nullptr; d.q_out = hq_out; d.s_out = hs_out;
        return hip_status(launch_gemv(d, st));
    }
    if (hipError_t e = launch_act_quant(x, dtype == BL_BF16, m, hidden, L.hp, nullptr, L.qx, L.sx, L.sumx, st))
        return hip_status(e);
    GemmProblem g{};
    g.qp = L.qx; g.kp = L.hp; g.s = L.sx; g.sumq = L.sumx; g.m = m; g.n = ffn;
    g.w0 = wg; g.w1 = wu; g.ldw = L.hp / 4; g.gamma0 = gate_gamma; g.gamma1 = up_gamma;
    g.out = L.h; g.acc_out = nullptr; g.epi = EPI_GATE;
    if (hipError_t e = launch_contraction(g, st)) return hip_status(e);
    float *sh = hs_out ? hs_out : L.sh;  // the requantization scales go straight to hs_out if asked
    if (hipError_t e = launch_act_quant(L.h, false, m, ffn, L.fp, hq_out, L.qh, sh, L.sumh, st))
        return hip_status(e);
    GemmProblem d{};
    d.qp = L.qh; d.kp = L.fp; d.s = sh; d.sumq = L.sumh; d.m = m; d.n = hidden;
    d.w0 = wd; d.w1 = nullptr; d.ldw = L.fp / 4; d.gamma0 = down_gamma; d.gamma1 = nullptr;
    d.out = y; d.acc_out = nullptr; d.epi = EPI_Y;
    return hip_status(launch_contraction(d, st));
}

}  // extern "C"
