// quantize.hip -- grouped dynamic quantization of BF16 rows (FP8 rowwise, MXFP8,
// MXFP4) and the standalone SwiGLU + MXFP4 requant, for gfx950.
//
// Both passes are HBM-bound streams.  One wave owns one row: each lane loads
// 16-byte vectors (8 bf16) so a wave reads 1 KiB per instruction, fully
// coalesced; all of a row's loads are issued before any is consumed.  MX block
// maxima are reduced across the 4 lanes that share a 32-element block; the
// rowwise maximum across the whole wave.  Codes are packed in registers and
// written as 8-byte (e4m3) or 4-byte (e2m1) stores per lane.
//
// (grouped_quantize_dynamic_scaled_fp4_async_kernel, description;
//  NvMxf4f8Strategy, grouped_quantize() / fused_silu_quantize().)
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;  // one row per wave
constexpr int kVecElems = 8;                     // bf16 per 16-byte vector
constexpr int kChunk = kWave * kVecElems;        // 512 elements per wave-wide load

__device__ __forceinline__ void load_offsets(uint32_t* s_off, const uint32_t* off, int G) {
    for (int i = threadIdx.x; i <= G; i += blockDim.x) s_off[i] = off[i];
    __syncthreads();
}

// ---------------------------------------------------------------------------
// FP8 rowwise: amax over the row, scale = amax / 448, code = e4m3(x / scale).
// NC = 16-byte vectors per lane held in registers (K <= NC * 512).
template <int NC>
__global__ __launch_bounds__(kThreads) void quantize_rowwise_kernel(const uint16_t* __restrict__ x,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ scales,
                                                                    const uint32_t* __restrict__ off, int G,
                                                                    int64_t T, int64_t K) {
    __shared__ uint32_t s_off[kMaxGroups + 1];
    load_offsets(s_off, off, G);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (t >= T || !wave_row_covered(s_off, G, T, t)) return;

    const int nvec = (int)(K / kVecElems);
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * K);
    uint4 v[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        int idx = c * kWave + lane;
        v[c] = idx < nvec ? xr[idx] : make_uint4(0, 0, 0, 0);
    }
    // bf16 magnitudes compare like their bit patterns with the sign cleared.
    uint32_t amax_bits = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax_bits = max(amax_bits, w[i] & 0x7fffu);
            amax_bits = max(amax_bits, (w[i] >> 16) & 0x7fffu);
        }
    }
    const float amax = wave_max(bf16_to_f32(amax_bits));
    const float scale = amax / 448.0f;  // IEEE binary32 division
    uint8_t* qr = q + t * K;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        int idx = c * kWave + lane;
        if (idx >= nvec) continue;
        float f[8];
        unpack8(v[c], f);
        uint32_t code[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            code[i] = amax == 0.0f ? (__float_as_uint(f[i]) >> 24) & 0x80u : enc_e4m3(f[i] / scale);
        uint2 packed;
        packed.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
        packed.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
        *reinterpret_cast<uint2*>(qr + (int64_t)idx * 8) = packed;
    }
    if (lane == 0) scales[t] = amax == 0.0f ? 0.0f : scale;
}

// Rows longer than the register budget: two passes over the row (the second
// one re-reads from cache).
__global__ __launch_bounds__(kThreads) void quantize_rowwise_long_kernel(const uint16_t* __restrict__ x,
                                                                         uint8_t* __restrict__ q,
                                                                         float* __restrict__ scales,
                                                                         const uint32_t* __restrict__ off,
                                                                         int G, int64_t T, int64_t K) {
    __shared__ uint32_t s_off[kMaxGroups + 1];
    load_offsets(s_off, off, G);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (t >= T || !wave_row_covered(s_off, G, T, t)) return;
    const int64_t nvec = K / kVecElems;
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * K);
    uint32_t amax_bits = 0;
    for (int64_t idx = lane; idx < nvec; idx += kWave) {
        uint4 v = xr[idx];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        for (int i = 0; i < 4; ++i) {
            amax_bits = max(amax_bits, w[i] & 0x7fffu);
            amax_bits = max(amax_bits, (w[i] >> 16) & 0x7fffu);
        }
    }
    const float amax = wave_max(bf16_to_f32(amax_bits));
    const float scale = amax / 448.0f;
    uint8_t* qr = q + t * K;
    for (int64_t idx = lane; idx < nvec; idx += kWave) {
        float f[8];
        unpack8(xr[idx], f);
        uint32_t code[8];
        for (int i = 0; i < 8; ++i)
            code[i] = amax == 0.0f ? (__float_as_uint(f[i]) >> 24) & 0x80u : enc_e4m3(f[i] / scale);
        uint2 packed;
        packed.x = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
        packed.y = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
        *reinterpret_cast<uint2*>(qr + idx * 8) = packed;
    }
    if (lane == 0) scales[t] = amax == 0.0f ? 0.0f : scale;
}

// U = vectors per lane loaded before any is encoded.
template <bool FP4, int U>
__global__ __launch_bounds__(kThreads) void quantize_mx_kernel(const uint16_t* __restrict__ x,
                                                               uint8_t* __restrict__ q,
                                                               uint8_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ off, int G, int64_t T,
                                                               int64_t K) {
    __shared__ uint32_t s_off[kMaxGroups + 1];
    load_offsets(s_off, off, G);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (t >= T || !wave_row_covered(s_off, G, T, t)) return;
    const int64_t nvec = K / kVecElems;
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * K);
    uint8_t* qrow = q + t * (FP4 ? K / 2 : K);
    uint8_t* srow = scales + t * (K / 32);
    for (int64_t base = 0; base < nvec; base += (int64_t)U * kWave) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t idx = base + u * kWave + lane;
            v[u] = idx < nvec ? xr[idx] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t idx = base + u * kWave + lane;
            // a block's 4 lanes are all in or all out (K is a multiple of 32),
            // so the shuffles inside mx_encode8 only mix lanes of one block
            float f[8];
            unpack8(v[u], f);
            uint32_t code[8];
            int X = mx_encode8<FP4>(f, code);
            if (idx < nvec) mx_store8<FP4>(code, X, qrow, srow, idx, lane);
        }
    }
}

// ---------------------------------------------------------------------------
// SwiGLU + MXFP4 requant of a BF16 [T, 2I] gate/up tensor.  A lane takes 8
// outputs (16 bf16 inputs, two 16-byte loads); 4 lanes form a 32-output block.
__global__ __launch_bounds__(kThreads) void silu_quantize_kernel(const uint16_t* __restrict__ h,
                                                                 uint8_t* __restrict__ yq,
                                                                 uint8_t* __restrict__ ys,
                                                                 const uint32_t* __restrict__ off, int G,
                                                                 int64_t T, int64_t I) {
    __shared__ uint32_t s_off[kMaxGroups + 1];
    load_offsets(s_off, off, G);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (t >= T || !wave_row_covered(s_off, G, T, t)) return;
    const int64_t nunits = I / 8;  // 8 outputs per lane-unit
    const uint4* hr = reinterpret_cast<const uint4*>(h + t * 2 * I);
    uint8_t* qrow = yq + t * (I / 2);
    uint8_t* srow = ys + t * (I / 32);
    for (int64_t base = 0; base < nunits; base += kWave) {
        const int64_t idx = base + lane;
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
        if (idx < nunits) {
            v0 = hr[2 * idx];
            v1 = hr[2 * idx + 1];
        }
        float gu[16];
        unpack8(v0, gu);
        unpack8(v1, gu + 8);
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = bf16_to_f32(f32_to_bf16(silu_mul(gu[2 * i], gu[2 * i + 1])));
        uint32_t code[8];
        int X = mx_encode8<true>(y, code);
        if (idx < nunits) mx_store8<true>(code, X, qrow, srow, idx, lane);
    }
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_quantize(int fmt, const void* x, void* q, void* scales, const uint32_t* off, int G, int64_t T,
                           int64_t K, hipStream_t stream) {
    const dim3 block(kThreads);
    const dim3 grid((unsigned)((T + kRowsPerBlock - 1) / kRowsPerBlock));
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint8_t* qb = static_cast<uint8_t*>(q);
    if (fmt == 0) {
        float* sf = static_cast<float*>(scales);
        const int64_t nc = (K + kChunk - 1) / kChunk;
        if (nc <= 1)
            hipLaunchKernelGGL(quantize_rowwise_kernel<1>, grid, block, 0, stream, xb, qb, sf, off, G, T, K);
        else if (nc <= 2)
            hipLaunchKernelGGL(quantize_rowwise_kernel<2>, grid, block, 0, stream, xb, qb, sf, off, G, T, K);
        else if (nc <= 4)
            hipLaunchKernelGGL(quantize_rowwise_kernel<4>, grid, block, 0, stream, xb, qb, sf, off, G, T, K);
        else if (nc <= 8)
            hipLaunchKernelGGL(quantize_rowwise_kernel<8>, grid, block, 0, stream, xb, qb, sf, off, G, T, K);
        else if (nc <= 14)
            hipLaunchKernelGGL(quantize_rowwise_kernel<14>, grid, block, 0, stream, xb, qb, sf, off, G, T, K);
        else if (nc <= 16)
            hipLaunchKernelGGL(quantize_rowwise_kernel<16>, grid, block, 0, stream, xb, qb, sf, off, G, T, K);
        else
            hipLaunchKernelGGL(quantize_rowwise_long_kernel, grid, block, 0, stream, xb, qb, sf, off, G, T, K);
    } else if (fmt == 1) {
        hipLaunchKernelGGL((quantize_mx_kernel<false, 7>), grid, block, 0, stream, xb, qb,
                           static_cast<uint8_t*>(scales), off, G, T, K);
    } else {
        hipLaunchKernelGGL((quantize_mx_kernel<true, 7>), grid, block, 0, stream, xb, qb,
                           static_cast<uint8_t*>(scales), off, G, T, K);
    }
    return hipGetLastError();
}

hipError_t launch_silu_quantize(const void* h, void* yq, void* ys, const uint32_t* off, int G, int64_t T,
                                int64_t I, hipStream_t stream) {
    const dim3 block(kThreads);
    const dim3 grid((unsigned)((T + kRowsPerBlock - 1) / kRowsPerBlock));
    hipLaunchKernelGGL(silu_quantize_kernel, grid, block, 0, stream, static_cast<const uint16_t*>(h),
                       static_cast<uint8_t*>(yq), static_cast<uint8_t*>(ys), off, G, T, I);
    return hipGetLastError();
}

}  // namespace mxg
