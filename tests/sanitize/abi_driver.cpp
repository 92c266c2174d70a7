// Drives every extern "C" entry point of libmxg's ABI layer (api.cpp) with
// the launchers replaced by recorders (abi_stubs.cpp): invalid arguments must
// return their documented status and launch nothing, valid ones must launch
// exactly once with the arguments passed through; the MXG_VALIDATE check runs
// on host arrays standing in for device memory.  Built with
// AddressSanitizer / UndefinedBehaviorSanitizer; exits 0 when every
// expectation holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "abi_stubs.h"
#include "mxg.h"

static int fails = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "expectation failed, line %d: %s\n", __LINE__, #cond); \
            ++fails;                                                   \
        }                                                              \
    } while (0)

// status and whether exactly one launch (of the named kind) happened
#define CALL(expected_status, launched, expr)                          \
    do {                                                               \
        const int before = g_stub.launches;                            \
        const mxg_status st_ = (expr);                                 \
        EXPECT(st_ == (expected_status));                              \
        EXPECT(g_stub.launches - before == ((launched) ? 1 : 0));      \
    } while (0)

int main() {
    // host buffers standing in for device tensors (256-byte aligned)
    std::vector<void*> owned;
    auto buf = [&owned](size_t n) {
        void* p = aligned_alloc(256, (n + 255) / 256 * 256);
        owned.push_back(p);
        return p;
    };
    const int64_t T = 64, K = 128, N = 96, I = 64, H = 64;
    const int G = 4, E = 3;
    void* x = buf(T * K * 2);
    void* q = buf(T * K);
    void* s = buf(T * K);
    void* b = buf(E * N * K);
    void* bs = buf(E * N * K);
    void* c = buf(T * N * 2);
    void* y = buf(T * H * 2);
    uint32_t* off = static_cast<uint32_t*>(buf(4 * (G + 1)));
    int32_t* ids = static_cast<int32_t*>(buf(4 * G));
    const uint32_t good_off[G + 1] = {0, 10, 10, 40, 64};
    const int32_t good_ids[G] = {0, 2, 1, 2};
    memcpy(off, good_off, sizeof good_off);
    memcpy(ids, good_ids, sizeof good_ids);
    char* odd = static_cast<char*>(x) + 1;
    char* four = static_cast<char*>(x) + 4;
    const mxg_format F8 = MXG_FP8_E4M3_ROWWISE, MX8 = MXG_MXFP8_E4M3, MX4 = MXG_MXFP4_E2M1;

    // ---- quantize family
    for (mxg_format f : {F8, MX8, MX4}) {
        CALL(MXG_SUCCESS, true, mx_grouped_quantize(f, x, q, s, off, ids, G, T, K, nullptr));
        EXPECT(strcmp(g_stub.last, "quantize") == 0);
        CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize(f, nullptr, q, s, off, ids, G, T, K, nullptr));
        CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize(f, odd, q, s, off, ids, G, T, K, nullptr));
        CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_quantize(f, x, q, s, off, ids, G, T, 40, nullptr));
        CALL(MXG_SUCCESS, false, mx_grouped_quantize(f, nullptr, nullptr, nullptr, nullptr, nullptr, G, 0, K, nullptr));
        CALL(MXG_SUCCESS, true, mx_grouped_quantize_gather(f, x, T, ids, 1, q, s, off, ids, G, T, K, nullptr));
        CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize_gather(f, x, T, ids, 0, q, s, off, ids, G, T, K, nullptr));
        CALL(MXG_SUCCESS, true, mx_grouped_quantize_scatter(f, x, 2, ids, 2, q, s, off, ids, G, T, K, nullptr));
        EXPECT(strcmp(g_stub.last, "quantize_scatter") == 0);
        CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize_scatter(f, x, 2, ids, 0, q, s, off, ids, G, T, K, nullptr));
        CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_quantize_scatter(f, x, 2, ids, 65, q, s, off, ids, G, T, K, nullptr));
        CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize_scatter(f, x, 2, nullptr, 2, q, s, off, ids, G, T, K, nullptr));
        CALL(MXG_SUCCESS, false, mx_grouped_quantize_scatter(f, nullptr, 0, nullptr, 2, q, s, off, ids, G, T, K, nullptr));
        CALL(MXG_ERROR_NOT_SUPPORTED, false,
             mx_grouped_quantize_scatter(f, x, (int64_t)INT32_MAX, ids, 2, q, s, off, ids, G, T, K, nullptr));
    }
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_quantize_scatter(F8, x, 2, ids, 2, q, s, off, ids, G, T, 8224, nullptr));
    CALL(MXG_SUCCESS, true, mx_grouped_quantize_scatter(MX4, x, 2, ids, 2, q, s, off, ids, G, T, 8224, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize((mxg_format)7, x, q, s, off, ids, G, T, K, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize(F8, x, q, s, off, ids, -1, T, K, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_quantize(F8, x, q, s, off, ids, MXG_MAX_GROUPS + 1, T, K, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize(F8, x, q, s, off, ids, G, T, -32, nullptr));
    const float sf[E] = {1.f, 2.f, 3.f};
    float* sfd = static_cast<float*>(buf(sizeof sf));
    memcpy(sfd, sf, sizeof sf);
    CALL(MXG_SUCCESS, true, mx_grouped_quantize_nvfp4(x, q, s, sfd, off, ids, G, E, T, K, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_quantize_nvfp4(x, q, s, sfd, off, ids, G, E, T, 24, nullptr));
    CALL(MXG_SUCCESS, true, mx_grouped_quantize_padded(MX4, x, q, s, off, 100, off, G, T, K, nullptr));
    CALL(MXG_SUCCESS, true, mx_grouped_quantize_nvfp4_padded(x, q, s, sfd, off, 100, off, ids, G, E, T, K, nullptr));
    EXPECT(strcmp(g_stub.last, "quantize_nvfp4_padded") == 0);
    CALL(MXG_ERROR_INVALID_VALUE, false,
         mx_grouped_quantize_nvfp4_padded(x, q, s, sfd, nullptr, 100, off, ids, G, E, T, K, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_quantize_padded(F8, x, q, s, off, 100, off, G, T, K, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize_padded(MX4, x, q, s, off, -1, off, G, T, K, nullptr));

    // ---- GEMMs
    CALL(MXG_SUCCESS, true, mx_grouped_matmul(F8, q, s, b, bs, c, off, ids, G, E, T, N, K, 17, nullptr));
    EXPECT(g_stub.gemm.fmt == 0 && g_stub.gemm.T == T && g_stub.gemm.N == N && g_stub.gemm.K == K &&
           g_stub.gemm.G == G && g_stub.gemm.E == E && g_stub.gemm.max_rows_hint == 17 && g_stub.gemm.yq == nullptr);
    CALL(MXG_SUCCESS, true, mx_grouped_matmul(MX4, q, s, b, bs, c, off, ids, G, E, T, N, K, 0, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_matmul(MX4, q, four, b, bs, c, off, ids, G, E, T, N, K, 0, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_matmul(MX8, q, s, b, four, c, off, ids, G, E, T, N, K, 0, nullptr));
    CALL(MXG_SUCCESS, true, mx_grouped_matmul(F8, q, four, b, four, c, off, ids, G, E, T, N, K, 0, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_matmul(F8, q, odd, b, bs, c, off, ids, G, E, T, N, K, 0, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false,
         mx_grouped_matmul(F8, q, s, b, bs, c, off, ids, G, E, T, (int64_t)INT32_MAX, K, 0, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false,
         mx_grouped_matmul(F8, q, s, b, bs, c, off, ids, G, E, (int64_t)INT32_MAX + 1, N, K, 0, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_matmul(F8, q, s, b, bs, c, off, ids, G, 0, T, N, K, 0, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false,
         mx_grouped_matmul(MX8, q, s, b, bs, c, off, ids, G, E, T, N, MXG_MAX_K + 512, 0, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false,
         mx_grouped_matmul_prepared(q, s, b, bs, c, off, ids, G, E, T, N, MXG_MAX_K + 512, nullptr));
    EXPECT(mxg_fp8_tile(G, T, N, K, 17, 1) == 256 && g_stub.gemm.b_prepared && g_stub.gemm.max_rows_hint == 17 &&
           g_stub.gemm.T == T && g_stub.gemm.N == N && g_stub.gemm.K == K && g_stub.gemm.fmt == 0);
    EXPECT(mxg_fp8_tile(0, T, N, K, 0, 0) == 0 && mxg_fp8_tile(G, T, N, 48, 0, 0) == 0 &&
           mxg_fp8_tile(G, T, N, MXG_MAX_K + 512, 0, 0) == 0 && mxg_fp8_tile(G, -1, N, K, 0, 0) == 0);
    CALL(MXG_SUCCESS, true, mx_grouped_matmul_prepared(q, s, b, bs, c, off, ids, G, E, T, N, K, nullptr));
    EXPECT(g_stub.gemm.b_prepared && g_stub.gemm.fmt == 0 && g_stub.gemm.b == b);
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_matmul_prepared(q, s, b, bs, c, off, ids, G, E, T, N, 96, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_matmul_prepared(q, s, odd, bs, c, off, ids, G, E, T, N, K, nullptr));
    CALL(MXG_SUCCESS, false, mx_grouped_matmul_prepared(q, s, b, bs, c, off, ids, G, E, 0, N, K, nullptr));
    EXPECT(mx_prepared_weights_bytes(E, N, K) == (int64_t)E * 256 * K);
    EXPECT(mx_prepared_weights_bytes(E, N, 96) == -1 && mx_prepared_weights_bytes(0, N, K) == -1);
    EXPECT(mx_prepared_weights_bytes(INT32_MAX, (int64_t)INT32_MAX / 2, (int64_t)INT32_MAX / 2 / 64 * 64) == -1);
    CALL(MXG_SUCCESS, true, mx_prepare_weights_fp8(b, E, N, K, bs, nullptr));
    EXPECT(strcmp(g_stub.last, "prepare_weights") == 0);
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_prepare_weights_fp8(b, E, N, 96, bs, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_prepare_weights_fp8(b, E, N, K, nullptr, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_prepare_weights_fp8(odd, E, N, K, bs, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_prepare_weights_fp8(b, 0, N, K, bs, nullptr));
    CALL(MXG_SUCCESS, true, mx_grouped_matmul_swiglu(MX4, q, s, b, bs, c, s, off, ids, G, E, T, I, K, 0, nullptr));
    EXPECT(g_stub.gemm.N == 2 * I && g_stub.gemm.yq == c);
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_matmul_swiglu(F8, q, s, b, bs, c, s, off, ids, G, E, T, I, K, 0, nullptr));
    CALL(MXG_SUCCESS, true, mx_grouped_matmul_padded(MX8, q, s, off, 100, b, bs, c, off, ids, G, E, T, N, K, 0, nullptr));
    EXPECT(g_stub.gemm.asoff == off && g_stub.gemm.as_rows == 100);
    CALL(MXG_SUCCESS, true,
         mx_grouped_matmul_swiglu_padded(MX4, q, s, off, 100, b, bs, c, s, off, ids, G, E, T, I, K, 0, nullptr));
    CALL(MXG_SUCCESS, true, mx_grouped_matmul_nvfp4(q, s, b, bs, sfd, c, off, ids, G, E, T, N, 512, 0, nullptr));
    CALL(MXG_SUCCESS, true,
         mx_grouped_matmul_nvfp4_padded(q, s, off, 100, b, bs, sfd, c, off, ids, G, E, T, N, 512, 0, nullptr));
    EXPECT(g_stub.gemm.fmt == 3 && g_stub.gemm.asoff == off && g_stub.gemm.as_rows == 100);
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_grouped_matmul_nvfp4(q, s, b, bs, sfd, c, off, ids, G, E, T, N, 256, 0, nullptr));
    CALL(MXG_SUCCESS, true,
         mx_grouped_matmul_swiglu_nvfp4(q, s, b, bs, sfd, nullptr, sfd, c, s, off, ids, G, E, T, I, 512, 0, nullptr));
    CALL(MXG_SUCCESS, true, mx_silu_quantize(y, q, s, off, G, T, I, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_silu_quantize(y, q, s, off, G, T, 40, nullptr));
    CALL(MXG_SUCCESS, true, mx_silu_quantize_nvfp4(y, q, s, sfd, off, ids, G, E, T, I, nullptr));

    // ---- combine and the clock probe
    CALL(MXG_SUCCESS, true, mx_moe_combine(y, T, H, ids, sfd, 2, 2, c, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_moe_combine(y, T, 12, ids, sfd, 2, 2, c, nullptr));
    CALL(MXG_ERROR_NOT_SUPPORTED, false, mx_moe_combine(y, T, H, ids, sfd, (int64_t)1 << 40, 64, c, nullptr));
    CALL(MXG_SUCCESS, false, mx_moe_combine(nullptr, T, H, ids, sfd, 0, 2, c, nullptr));
    CALL(MXG_SUCCESS, true, mxg_clock_probe(static_cast<unsigned long long*>(buf(16)), 1000, nullptr));
    CALL(MXG_ERROR_INVALID_VALUE, false, mxg_clock_probe(static_cast<unsigned long long*>(buf(16)), 0, nullptr));

    // ---- MXG_VALIDATE: routing copied to the host and checked before any launch
    setenv("MXG_VALIDATE", "1", 1);
    const int copies0 = g_stub.copies;
    CALL(MXG_SUCCESS, true, mx_grouped_matmul(F8, q, s, b, bs, c, off, ids, G, E, T, N, K, 0, nullptr));
    EXPECT(g_stub.copies - copies0 == 2);
    EXPECT(strcmp(mxg_validation_message(), "") == 0);
    const uint32_t bad_off[G + 1] = {0, 10, 9, 40, 64};
    memcpy(off, bad_off, sizeof bad_off);
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_matmul(F8, q, s, b, bs, c, off, ids, G, E, T, N, K, 0, nullptr));
    EXPECT(strstr(mxg_validation_message(), "below") != nullptr);
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize(MX4, x, q, s, off, ids, G, T, K, nullptr));
    memcpy(off, good_off, sizeof good_off);
    ids[3] = E;
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_matmul(F8, q, s, b, bs, c, off, ids, G, E, T, N, K, 0, nullptr));
    EXPECT(strstr(mxg_validation_message(), "expert_ids[3]") != nullptr);
    CALL(MXG_SUCCESS, true, mx_grouped_quantize(F8, x, q, s, off, ids, G, T, K, nullptr));  // ids not read here
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_grouped_quantize_nvfp4(x, q, s, sfd, off, ids, G, E, T, K, nullptr));
    off[4] = (uint32_t)T + 1;
    CALL(MXG_ERROR_INVALID_VALUE, false, mx_silu_quantize(y, q, s, off, G, T, I, nullptr));
    unsetenv("MXG_VALIDATE");
    CALL(MXG_SUCCESS, true, mx_silu_quantize(y, q, s, off, G, T, I, nullptr));  // not checked without it

    // ---- the host check itself, including short message buffers
    char msg[8];
    EXPECT(mxg_routing_violation(good_off, good_ids, G, E, T, msg, sizeof msg) == 0 && msg[0] == 0);
    EXPECT(mxg_routing_violation(bad_off, good_ids, G, E, T, msg, sizeof msg) == 1 && strlen(msg) == 7);
    EXPECT(mxg_routing_violation(bad_off, good_ids, G, E, T, nullptr, 0) == 1);
    EXPECT(mxg_routing_violation(bad_off, good_ids, G, E, T, msg, 1) == 1 && msg[0] == 0);
    EXPECT(mxg_routing_violation(nullptr, good_ids, G, E, T, msg, sizeof msg) == -1);
    for (int st = -1; st <= 4; ++st) EXPECT(mxg_status_string((mxg_status)st) != nullptr);

    for (void* p : owned) free(p);
    printf("launches %d copies %d fails %d\n", g_stub.launches, g_stub.copies, fails);
    return fails == 0 ? 0 : 1;
}
