// clock.hip -- shader-clock probe for measurement: one wave counts the
// shader-clock counter against the constant 100 MHz counter while it sleeps,
// so the ratio is the average engine clock over that window.  Launched on a
// stream of its own beside a timed region, it measures the clock the other
// kernels run at (it occupies one wave slot of one CU and issues almost
// nothing).  Device code for gfx950.
#include "mxg_internal.h"

namespace mxg {

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out, unsigned long long ticks) {
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();  // 100 MHz
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();      // shader clock
    unsigned long long r = r0;
    while (r - r0 < ticks) {
        __builtin_amdgcn_s_sleep(64);
        r = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    // every lane stores (vector stores); lanes 0 and 1 hold the two results
    const int lane = threadIdx.x;
    if (lane < 2) out[lane] = lane == 0 ? c1 - c0 : r - r0;
}

}  // namespace

hipError_t launch_clock_probe(unsigned long long* out, unsigned long long ticks, hipStream_t stream) {
    hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, ticks);
    return hipGetLastError();
}

}  // namespace mxg
