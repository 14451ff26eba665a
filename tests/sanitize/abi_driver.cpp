// Drives the host-side argument checks of the C ABI (include/bitlinear.h) under
// AddressSanitizer and UndefinedBehaviorSanitizer, host code only (built and run
// by tests/test_sanitizers.py). Every call here is rejected before anything is
// enqueued, so no GPU is needed; the size queries run at the largest shapes the
// boundary accepts, where the workspace arithmetic is widest.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "../../include/bitlinear.h"

static int failures = 0;
#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++failures; } } while (0)

int main()
{
    void *A = reinterpret_cast<void *>(0x10000);  // aligned fake device address, never dereferenced
    void *MIS = reinterpret_cast<void *>(0x10004);
    const int64_t big = BL_MAX_DIM, tok = BL_MAX_TOKENS;
    for (int op = -1; op <= 9; ++op) {
        (void)bitlinear_workspace_size(op, tok, big, big);
        (void)bitlinear_workspace_size(op, 1, 4, 1);
        (void)bitlinear_workspace_size(op, 0, 0, 0);
        (void)bitlinear_workspace_size(op, -5, -4, -1);
        (void)bitlinear_workspace_size(op, std::numeric_limits<int64_t>::max(), big, big);
    }
    CHECK(bitlinear_workspace_size(BL_OP_FORWARD, tok, big, big) > 0);
    CHECK(bitlinear_workspace_size(BL_OP_FORWARD, tok + 1, big, big) == 0);
    for (int s = -1; s <= 9; ++s) CHECK(bitlinear_status_string(static_cast<bl_status>(s)) != nullptr);

    auto f32 = static_cast<const float *>(A);
    auto u8 = static_cast<const uint8_t *>(A);
    CHECK(bitlinear_forward(nullptr, BL_BF16, 1, 256, u8, f32, 8, (float *)A, nullptr, nullptr, 0, nullptr) == BL_ERR_NULL);
    CHECK(bitlinear_forward(A, (bl_dtype)7, 1, 256, u8, f32, 8, (float *)A, nullptr, nullptr, 0, nullptr) == BL_ERR_DTYPE);
    CHECK(bitlinear_forward(A, BL_BF16, tok + 1, 256, u8, f32, 8, (float *)A, nullptr, nullptr, 0, nullptr) == BL_ERR_SHAPE);
    CHECK(bitlinear_forward(A, BL_BF16, 1, big + 4, u8, f32, 8, (float *)A, nullptr, nullptr, 0, nullptr) == BL_ERR_SHAPE);
    CHECK(bitlinear_forward(MIS, BL_BF16, 1, 256, u8, f32, 8, (float *)A, nullptr, nullptr, 0, nullptr) == BL_ERR_ALIGN);
    CHECK(bitlinear_forward(A, BL_BF16, 64, 256, u8, f32, 8, (float *)A, nullptr, A, 16, nullptr) == BL_ERR_WORKSPACE);
    CHECK(bitlinear_forward_noalloc(A, BL_BF16, tok, big, u8, f32, 8, (float *)A, nullptr, nullptr) == BL_ERR_WORKSPACE);
    CHECK(bitlinear_forward_norm(A, BL_BF16, 1, 256, (const float *)MIS, u8, f32, 8, (float *)A, nullptr, A,
                                 1 << 20, nullptr) == BL_ERR_ALIGN);
    CHECK(bitlinear_forward_a4(A, BL_BF16, 1, 256, 0, u8, f32, 8, (float *)A, nullptr, A, 1 << 20, nullptr) == BL_ERR_VALUE);
    CHECK(bitlinear_forward_a4(A, BL_BF16, 1, 256, 257, u8, f32, 8, (float *)A, nullptr, A, 1 << 20, nullptr) == BL_ERR_VALUE);
    CHECK(bitlinear_quant_act(A, BL_F32, 1, 2, (int8_t *)A, (float *)A, nullptr) == BL_ERR_SHAPE);
    CHECK(bitlinear_quant_act_norm(A, BL_F32, 1, 256, f32, (int8_t *)MIS, (float *)A, nullptr) == BL_ERR_ALIGN);
    CHECK(bitlinear_quant_act_a4(A, BL_F32, 1, 256, -1, (int8_t *)A, (float *)A, nullptr) == BL_ERR_VALUE);
    CHECK(bitlinear_pack_weights(f32, 8, 255, (uint8_t *)A, (float *)A, A, 1 << 20, nullptr) == BL_ERR_SHAPE);
    CHECK(bitlinear_pack_weights_threshold(f32, 8, 256, std::nanf(""), (uint8_t *)A, (float *)A, nullptr, A,
                                           1 << 20, nullptr) == BL_ERR_VALUE);
    CHECK(bitlinear_pack_weights_threshold(f32, 8, 256, -1.0f, (uint8_t *)A, (float *)A, nullptr, A, 1 << 20,
                                           nullptr) == BL_ERR_VALUE);
    CHECK(bitlinear_pack_kmajor(u8, 6, 256, (uint8_t *)A, nullptr) == BL_ERR_SHAPE);
    CHECK(bitlinear_gemm_i32((const int8_t *)A, 4, 256, u8, 8, (int32_t *)A, A, 0, nullptr) == BL_ERR_WORKSPACE);
    CHECK(bitlinear_ffn(A, BL_BF16, 1, 256, 510, u8, f32, u8, f32, u8, f32, (float *)A, nullptr, nullptr, A,
                        1 << 20, nullptr) == BL_ERR_SHAPE);
    CHECK(bitlinear_ffn_sparse(A, BL_BF16, 5, 4096, 14336, u8, f32, u8, f32, u8, f32, (float *)A, nullptr,
                               nullptr, A, 1 << 20, nullptr) == BL_ERR_SHAPE);
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi driver: ok\n");
    return 0;
}
