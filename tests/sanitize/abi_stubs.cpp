// Host-only stand-ins for everything libmxg's C ABI layer calls below it: the
// kernel launchers (they record the call instead of launching) and the two
// HIP runtime calls the MXG_VALIDATE check makes (a device-to-host copy and a
// stream synchronise; here the "device" pointers are host memory).  Linked
// with api.cpp into a sanitizer build that needs no GPU.
#include <string.h>

#include "mxg_internal.h"
#include "abi_stubs.h"

StubLog g_stub;

namespace mxg {

static hipError_t record(const char* what) {
    ++g_stub.launches;
    g_stub.last = what;
    return hipSuccess;
}

hipError_t launch_quantize(int, const void*, void*, void*, const uint32_t*, int, int64_t, int64_t, hipStream_t) {
    return record("quantize");
}
hipError_t launch_quantize_gather(int, const void*, int64_t, const int32_t*, int32_t, void*, void*, const uint32_t*,
                                  int, int64_t, int64_t, hipStream_t) {
    return record("quantize_gather");
}
hipError_t launch_quantize_scatter(int, const void*, int64_t, const int32_t*, int, void*, void*, const uint32_t*, int,
                                   int64_t, int64_t, hipStream_t) {
    return record("quantize_scatter");
}
hipError_t launch_quantize_padded(int, const void*, void*, void*, const uint32_t*, int64_t, const uint32_t*, int,
                                  int64_t, int64_t, hipStream_t) {
    return record("quantize_padded");
}
hipError_t launch_quantize_nvfp4(const void*, void*, void*, const float*, const uint32_t*, const int32_t*, int, int,
                                 int64_t, int64_t, hipStream_t) {
    return record("quantize_nvfp4");
}
hipError_t launch_quantize_nvfp4_padded(const void*, void*, void*, const float*, const uint32_t*, int64_t,
                                        const uint32_t*, const int32_t*, int, int, int64_t, int64_t, hipStream_t) {
    return record("quantize_nvfp4_padded");
}
hipError_t launch_combine(const void*, int64_t, int64_t, const int32_t*, const float*, int64_t, int, void*,
                          hipStream_t) {
    return record("combine");
}
hipError_t launch_silu_quantize(const void*, void*, void*, const uint32_t*, int, int64_t, int64_t, hipStream_t) {
    return record("silu_quantize");
}
hipError_t launch_silu_quantize_nvfp4(const void*, void*, void*, const float*, const uint32_t*, const int32_t*, int,
                                      int, int64_t, int64_t, hipStream_t) {
    return record("silu_quantize_nvfp4");
}
hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t) {
    g_stub.gemm = p;
    return record("grouped_gemm");
}
hipError_t launch_clock_probe(unsigned long long*, unsigned long long, hipStream_t) { return record("clock_probe"); }
int64_t prepared_weights_bytes(int64_t E, int64_t N, int64_t K) { return E * ((N + 255) / 256) * 256 * K; }
int fp8_tile_choice(const GemmProblem& p) {
    g_stub.gemm = p;
    return 256;
}
hipError_t launch_prepare_weights(const void*, int64_t, int64_t, int64_t, void*, hipStream_t) {
    return record("prepare_weights");
}

}  // namespace mxg

extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
    memcpy(dst, src, bytes);
    ++g_stub.copies;
    return hipSuccess;
}

extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
