// Host-side checks of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code: the workspace-size queries over a grid of shapes (extreme ones
// included), and calls that fail their host checks before anything is enqueued (no GPU is
// needed and none is touched). Exit status 0 when every documented status comes back.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "vsa.h"

static int g_fails = 0;
#define EXPECT(c)                                                                       \
    do {                                                                                \
        if (!(c)) {                                                                     \
            std::printf("FAIL line %d: %s\n", __LINE__, #c);                            \
            ++g_fails;                                                                  \
        }                                                                               \
    } while (0)

static void* const F = reinterpret_cast<void*>(0x100000);          // never dereferenced
static void* const W = reinterpret_cast<void*>(0x100000 * 256);    // 256-byte aligned

static vsa_status attention(const void* q, int dtype, int B, int total, int hq, int hkv, int d,
                            int s_max, int rows, int mkv, float scale, uint32_t flags,
                            void* ws, size_t ws_bytes) {
    return verify_attention(q, F, F, (vsa_dtype)dtype, (const int32_t*)F, (const int32_t*)F, B,
                            total, hq, hkv, d, s_max, rows, mkv, scale, flags, (float*)F, ws, ws_bytes,
                            nullptr);
}

static vsa_status sample(const float* target, const int32_t* drafts, int B, int total, int V,
                         int rows, int mtk, int mtl, void* ws, size_t ws_bytes) {
    return verify_sample_accept(target, (const float*)F, drafts, (const int32_t*)F, nullptr,
                                (const vsa_row_params*)F, (const int32_t*)F, 0, B, total, V,
                                rows, mtk, mtl, (int32_t*)F, (int32_t*)F, nullptr, nullptr,
                                nullptr, nullptr, nullptr, ws, ws_bytes, nullptr);
}

int main() {
    EXPECT(vsa_version() > 0);
    for (int s = 0; s < 8; ++s) EXPECT(vsa_status_string((vsa_status)s) != nullptr);

    // ---- workspace sizes over a grid of shapes, extreme values included
    const int ints[] = {INT_MIN, -1, 0, 1, 2, 3, 4, 31, 32, 33, 64, 127, 128, 129, 255, 256,
                        257, 1024, 2048, 2049, 16384, 65536, 151936, 262144, 524288, 524289,
                        1 << 24, INT_MAX / 3, INT_MAX / 2, INT_MAX - 1, INT_MAX};
    size_t sink = 0;
    for (int b : ints)
        for (int r : {0, 1, 5, 32, 33})
            for (int v : ints) {
                sink += verify_attention_workspace_size(b, 32, 8, 128, r, v);
                sink += verify_attention_workspace_size(b, 8, 8, 64, r, v);
                sink += verify_sample_accept_workspace_size(b, b * 0 + r, v, r, 20, 5);
                sink += verify_sample_accept_workspace_size(b, INT_MAX, v, r, 256, 32);
                sink += verify_sample_accept_workspace_size(b, v, 151936, 32, r, r);
                sink += small_m_qmm_workspace_size(r, v, b);
            }
    for (int hq : ints)
        for (int hkv : ints) sink += verify_attention_workspace_size(4, hq, hkv, 128, 5, 8197);
    std::printf("sizes checksum %zu\n", sink);
    const size_t ok = verify_attention_workspace_size(4, 32, 8, 128, 5, 8197);
    EXPECT(ok > 0 && ok % 256 == 0);
    EXPECT(verify_attention_workspace_size(4, 30, 8, 128, 5, 8197) == 0);
    EXPECT(verify_attention_workspace_size(4, 32, 8, 96, 5, 8197) == 0);
    EXPECT(verify_attention_workspace_size(0, 32, 8, 128, 5, 8197) == 0);
    EXPECT(verify_sample_accept_workspace_size(4, 20, 151936, 5, 0, 0) > 0);
    EXPECT(verify_sample_accept_workspace_size(4, 20, 151936, 5, 257, 0) == 0);
    EXPECT(verify_sample_accept_workspace_size(4, 3, 151936, 5, 0, 0) == 0);

    // ---- calls that fail a host check
    EXPECT(attention(nullptr, VSA_BF16, 4, 20, 32, 8, 128, 8256, 5, 8197, 0.f, 0, W, 1u << 30) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(attention(F, 7, 4, 20, 32, 8, 128, 8256, 5, 8197, 0.f, 0, W, 1u << 30) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(attention(F, VSA_BF16, 4, 41, 32, 8, 128, 8256, 5, 8197, 0.f, 0, W, 1u << 30) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(attention(F, VSA_BF16, 4, 20, 32, 8, 128, 8256, 5, 8197,
                     std::numeric_limits<float>::quiet_NaN(), 0, W, 1u << 30) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(attention(F, VSA_BF16, 4, 20, 32, 8, 96, 8256, 5, 8197, 0.f, 0, W, 1u << 30) ==
           VSA_ERR_UNSUPPORTED);
    EXPECT(attention(F, VSA_BF16, INT_MAX, INT_MAX, 32, 8, 128, INT_MAX, 32, INT_MAX, 0.f, 0, W,
                     1u << 30) != VSA_OK);
    EXPECT(attention(F, VSA_BF16, 4, 20, 32, 8, 128, 8256, 5, 8197, 0.f, 0, nullptr, 1u << 30) ==
           VSA_ERR_WORKSPACE);
    EXPECT(attention(F, VSA_BF16, 4, 20, 32, 8, 128, 8256, 5, 8197, 0.f, 0, W, 1024) ==
           VSA_ERR_WORKSPACE);
    EXPECT(sample(nullptr, (const int32_t*)F, 4, 20, 151936, 5, 0, 0, W, 1u << 30) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(sample((const float*)F, nullptr, 4, 20, 151936, 5, 0, 0, W, 1u << 30) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(sample((const float*)F, (const int32_t*)F, 4, 20, 1 << 30, 5, 0, 0, W, 1u << 30) ==
           VSA_ERR_UNSUPPORTED);
    EXPECT(sample((const float*)F, (const int32_t*)F, INT_MAX, INT_MAX, 524288, 32, 256, 32, W,
                  1u << 30) != VSA_OK);
    EXPECT(sample((const float*)F, (const int32_t*)F, 4, 20, 151936, 5, 0, 0, nullptr,
                  1u << 30) == VSA_ERR_WORKSPACE);
    EXPECT(sample((const float*)F, (const int32_t*)F, 4, 20, 151936, 5, 0, 0, W, 256) ==
           VSA_ERR_WORKSPACE);
    EXPECT(draft_vocab_inverse(nullptr, 10, 100, (int32_t*)W, nullptr) == VSA_ERR_INVALID_ARG);
    EXPECT(draft_vocab_inverse((const int32_t*)F, 101, 100, (int32_t*)W, nullptr) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(small_m_qmm(nullptr, (const uint8_t*)W, W, 4, 8, 1024, 4096, (float*)W, W, 1u << 30,
                       nullptr) == VSA_ERR_INVALID_ARG);
    EXPECT(small_m_qmm(W, (const uint8_t*)W, W, 4, 17, 1024, 4096, (float*)W, W, 1u << 30, nullptr) ==
           VSA_ERR_UNSUPPORTED);
    EXPECT(small_m_qmm(W, (const uint8_t*)W, W, 4, 8, 1024, 1 << 30, (float*)W, W, 1u << 30,
                       nullptr) == VSA_ERR_UNSUPPORTED);
    EXPECT(small_m_qmm(W, (const uint8_t*)W, W, 4, 8, 1024, 4096, (float*)W + 1, W, 1u << 30,
                       nullptr) == VSA_ERR_INVALID_ARG);
    const int32_t* I = (const int32_t*)F;
    EXPECT(verify_attention_noalloc(nullptr, F, F, VSA_BF16, I, I, 4, 20, 32, 8, 128, 8256, 5,
                                    8197, 0.f, 0, (float*)F, nullptr, nullptr) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(verify_attention_noalloc(F, F, F, VSA_BF16, I, I, 65536, 65536, 64, 8, 128,
                                    INT_MAX, 32, INT_MAX, 0.f, 0, (float*)F, nullptr,
                                    nullptr) != VSA_OK);
    EXPECT(block_attention(F, F, F, VSA_BF16, I, I, 4, 20, 32, 8, 128, 8256, 5, 8197, 0.f, -1,
                           0, (float*)F, W, 1u << 30, nullptr) == VSA_ERR_INVALID_ARG);
    EXPECT(block_attention(F, F, F, VSA_BF16, I, I, 4, 20, 32, 8, 128, 8256, 5, 8197, 0.f, 0,
                           0x80u, (float*)F, W, 1u << 30, nullptr) == VSA_ERR_INVALID_ARG);
    EXPECT(block_attention(F, F, F, VSA_BF16, I, I, 1 << 20, 1 << 20, 32, 8, 128, 8256, 5, 8197,
                           0.f, 0, 0, (float*)F, W, 1u << 30, nullptr) == VSA_ERR_UNSUPPORTED);
    const uint8_t* U = (const uint8_t*)F;
    EXPECT(verify_attention_kvq(F, U, F, U, F, 5, I, I, 4, 20, 32, 8, 128, 8256, 5, 8197, 0.f, 0,
                                (float*)F, W, 1u << 30, nullptr) == VSA_ERR_INVALID_ARG);
    EXPECT(verify_attention_kvq(F, U, F, U, F, 8, I, I, INT_MAX, INT_MAX, INT_MAX, 1, 128,
                                INT_MAX, 32, INT_MAX, 0.f, 0, (float*)F, W, 1u << 30,
                                nullptr) != VSA_OK);
    EXPECT(verify_sample_accept_reduced_draft(
               (const float*)F, (const float*)F, 151937, I, I, I, nullptr,
               (const vsa_row_params*)F, I, 0, 4, 20, 151936, 5, 0, 0, (int32_t*)F,
               (int32_t*)F, nullptr, nullptr, nullptr, nullptr, nullptr, W, 1u << 30,
               nullptr) == VSA_ERR_INVALID_ARG);
    EXPECT(verify_sample_accept_reduced_draft(
               (const float*)F, (const float*)F, 32000, nullptr, I, I, nullptr,
               (const vsa_row_params*)F, I, 0, 4, 20, 151936, 5, 0, 0, (int32_t*)F,
               (int32_t*)F, nullptr, nullptr, nullptr, nullptr, nullptr, W, 1u << 30,
               nullptr) == VSA_ERR_INVALID_ARG);
    EXPECT(verify_sample_accept_onehot((const float*)F, nullptr, I, nullptr,
                                       (const vsa_row_params*)F, I, 0, 4, 20, 151936, 5, 0, 0,
                                       (int32_t*)F, (int32_t*)F, nullptr, nullptr, nullptr,
                                       nullptr, nullptr, W, 1u << 30, nullptr) ==
           VSA_ERR_INVALID_ARG);
    EXPECT(verify_sample_accept_onehot((const float*)F, I, I, nullptr, (const vsa_row_params*)F,
                                       I, 0, 1 << 23, 1 << 23, 151936, 5, 0, 0, (int32_t*)F,
                                       (int32_t*)F, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       W, 1u << 30, nullptr) == VSA_ERR_UNSUPPORTED);
    EXPECT(verify_sample_accept_workspace_size(1 << 23, 1 << 23, 151936, 5, 0, 0) == 0);
    EXPECT(verify_sample_accept_workspace_size(200000, 600000, 8, 3, 0, 0) > 0);
    EXPECT(verify_attention_workspace_size(65536, 128, 128, 128, 1, 8192) == 0);
    EXPECT(small_m_qmm_workspace_size(8, 1024, 1 << 30) == 0);
    // grids beyond one dispatch (2^24 - 1 workgroups of 256 threads) are refused
    EXPECT(verify_sample_accept_workspace_size(1 << 22, 1 << 22, 524288, 1, 0, 0) == 0);
    EXPECT(verify_sample_accept_workspace_size(1 << 22, 1 << 22, 2048, 1, 0, 0) > 0);
    EXPECT(sample((const float*)F, (const int32_t*)F, 1 << 22, 1 << 22, 524288, 1, 0, 0, W,
                  1u << 30) == VSA_ERR_UNSUPPORTED);
    EXPECT(small_m_qmm_workspace_size(8, INT_MAX, 4096) == 0);
    EXPECT(small_m_qmm(W, (const uint8_t*)W, W, 4, 8, INT_MAX, 4096, (float*)W, W, 1u << 30,
                       nullptr) == VSA_ERR_UNSUPPORTED);
    std::printf("%s (%d failures)\n", g_fails ? "FAILED" : "ok", g_fails);
    return g_fails ? 1 : 0;
}
