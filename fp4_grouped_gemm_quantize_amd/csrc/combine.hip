// combine.hip -- MoE combine after the down-projection, for gfx950: each token's
// output row is the router-weighted sum of the expert rows its slots were
// routed to.
//
// (grouped_matmul_rowwise_dynamic_scaled_fp8, Parameters: elementwise_lambda_fn
//  -- the optional output epilogue at (global_row, n) where this weighting and
//  the combine attach; NvMxf4f8Strategy, prepare_swiglu_operands(): the
//  EP-combine path; Struct_ep_dispatch_mxfp4: src_info, the source of each
//  dispatched row.)
//
// Design: a gather-sum per token instead of a scatter-add from the GEMM
// epilogue -- no atomics, no fp32 staging buffer, a fixed summation order
// (slot k = 0, 1, ...), so the result is deterministic.  One wave per token;
// each lane owns 8 consecutive outputs (16-byte loads of BF16 rows) per
// 512-wide chunk of H and keeps fp32 sums; the slot table is read by the
// lanes 64 entries at a time and broadcast with shuffles.  HBM traffic is the
// routed rows once plus the output once.
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kGather = 8;  // slot rows loaded together per lane

__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ y, int64_t T, int64_t H,
                                                           const int32_t* __restrict__ row_of_slot,
                                                           const float* __restrict__ wts, int64_t ntok, int top_k,
                                                           uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (t >= ntok) return;
    const int64_t nunits = H / 8;
    const int32_t* slots = row_of_slot + t * top_k;
    const float* wt = wts + t * top_k;
    for (int64_t base = 0; base < nunits; base += kWave) {
        const int64_t u = base + lane;
        const bool on = u < nunits;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < top_k; k0 += kWave) {
            const int kk = k0 + lane;
            int32_t r = -1;
            float wk = 0.0f;
            if (kk < top_k) {
                r = slots[kk];
                wk = wt[kk];
            }
            const int kn = top_k - k0 < kWave ? top_k - k0 : kWave;
            // slots in groups of kGather: all their row loads are issued
            // before any is accumulated (one load at a time left each wave
            // waiting out the memory latency per slot); the accumulation
            // order stays slot 0, 1, ...
            for (int j0 = 0; j0 < kn; j0 += kGather) {
                uint4 v[kGather];
                float wj[kGather];
                bool use[kGather];
#pragma unroll
                for (int q = 0; q < kGather; ++q) {
                    const int j = j0 + q < kn ? j0 + q : 0;  // uniform
                    const int32_t rj = __shfl(r, j, kWave);
                    wj[q] = __shfl(wk, j, kWave);
                    use[q] = j0 + q < kn && rj >= 0 && (int64_t)rj < T;  // wave-uniform: a dropped slot
                    v[q] = use[q] && on ? *reinterpret_cast<const uint4*>(y + (int64_t)rj * H + u * 8)
                                        : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int q = 0; q < kGather; ++q) {
                    if (!use[q] || !on) continue;
                    float f[8];
                    unpack8(v[q], f);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[q], f[i], acc[i]);
                }
            }
        }
        if (on) {
            uint4 o;
            o.x = f32x2_to_bf16x2(acc[0], acc[1]);
            o.y = f32x2_to_bf16x2(acc[2], acc[3]);
            o.z = f32x2_to_bf16x2(acc[4], acc[5]);
            o.w = f32x2_to_bf16x2(acc[6], acc[7]);
            *reinterpret_cast<uint4*>(out + t * H + u * 8) = o;
        }
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int64_t T, int64_t H, const int32_t* row_of_slot, const float* weights,
                          int64_t ntok, int top_k, void* out, hipStream_t stream) {
    const int64_t blocks = (ntok + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(y), T, H, row_of_slot, weights, ntok, top_k,
                       static_cast<uint16_t*>(out));
    return hipGetLastError();
}

}  // namespace mxg
