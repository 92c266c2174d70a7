// mxg_internal.h -- launchers the C ABI layer calls; host-side only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

hipError_t launch_quantize(int fmt, const void* x, void* q, void* scales, const uint32_t* off, int G, int64_t T,
                           int64_t K, hipStream_t stream);

// The same with row t read from row indices[t] / divisor of x (nsrc rows).
hipError_t launch_quantize_gather(int fmt, const void* x, int64_t nsrc, const int32_t* indices, int32_t divisor,
                                  void* q, void* scales, const uint32_t* off, int G, int64_t T, int64_t K,
                                  hipStream_t stream);

// Token-major form: token row s (of ntok) is quantized once into every routed row
// row_of_slot[s * top_k + k] in [0, T) that a group covers (top_k <= 64; FP8 rowwise K <= 8192).
hipError_t launch_quantize_scatter(int fmt, const void* x, int64_t ntok, const int32_t* row_of_slot, int top_k,
                                   void* q, void* scales, const uint32_t* off, int G, int64_t T, int64_t K,
                                   hipStream_t stream);

// MX (fmt 1, 2) with group g's scales from row scales_offsets[g] of a [scale_rows, K/32] tensor.
hipError_t launch_quantize_padded(int fmt, const void* x, void* q, void* scales, const uint32_t* scales_offsets,
                                  int64_t scale_rows, const uint32_t* off, int G, int64_t T, int64_t K,
                                  hipStream_t stream);

// NVFP4: rows of group g use tensor_scales[ids[g]]; groups with an id outside [0, E) are skipped.
hipError_t launch_quantize_nvfp4(const void* x, void* q, void* scales, const float* tensor_scales,
                                  const uint32_t* off, const int32_t* ids, int G, int E, int64_t T, int64_t K,
                                  hipStream_t stream);

// NVFP4 with group g's E4M3 scales from row scales_offsets[g] of a [scale_rows, K/16] tensor.
hipError_t launch_quantize_nvfp4_padded(const void* x, void* q, void* scales, const float* tensor_scales,
                                        const uint32_t* scales_offsets, int64_t scale_rows, const uint32_t* off,
                                        const int32_t* ids, int G, int E, int64_t T, int64_t K, hipStream_t stream);

// out[t, :] = bf16(sum_k weights[t*top_k + k] * y[row_of_slot[t*top_k + k], :]).
hipError_t launch_combine(const void* y, int64_t T, int64_t H, const int32_t* row_of_slot, const float* weights,
                          int64_t ntok, int top_k, void* out, hipStream_t stream);

hipError_t launch_silu_quantize(const void* h, void* yq, void* ys, const uint32_t* off, int G, int64_t T,
                                int64_t I, hipStream_t stream);

// NVFP4 requant of y = bf16(silu(g) u): rows of group g use y_scales_sf[ids[g]].
hipError_t launch_silu_quantize_nvfp4(const void* h, void* yq, void* ys, const float* y_sf, const uint32_t* off,
                                      const int32_t* ids, int G, int E, int64_t T, int64_t I, hipStream_t stream);

// Grouped GEMM; when yq != nullptr the SwiGLU + MXFP4 requant epilogue runs
// (N = 2I) and c is not written.
struct GemmProblem {
    int fmt;
    const void* a;
    const void* a_scales;
    const void* b;
    const void* b_scales;
    void* c;
    void* yq;
    void* ys;
    const uint32_t* off;
    const int32_t* ids;
    int G;
    int E;
    int64_t T;
    int64_t N;
    int64_t K;
    int64_t max_rows_hint;
    const float* es;   // NVFP4 (fmt 3): per-expert epilogue scale, fp32 [E]
    const void* rs;    // NVFP4 fused: optional bf16 row scales [T]
    const float* ysf;  // NVFP4 fused: per-expert encode-side tensor scale of y, fp32 [E]
    const uint32_t* asoff;  // padded A scales: group g's rows from row asoff[g] (nullptr: dense)
    int64_t as_rows;        // rows of that scale tensor
    bool b_prepared;        // FP8 rowwise: b holds the prepared weights (launch_prepare_weights)
};

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream);

// The FP8 rowwise tile launch_grouped_gemm runs for p: 384 or 256 (256-row
// tiles of that many columns), 32 (the 32 x 256 decode tile), 0 otherwise.
int fp8_tile_choice(const GemmProblem& p);

// FP8 rowwise weights [E, N, K] (K a multiple of 64) into the layout the
// GEMM's 64-byte-stage rings load as it is; out holds prepared_weights_bytes(E, N, K).
int64_t prepared_weights_bytes(int64_t E, int64_t N, int64_t K);
hipError_t launch_prepare_weights(const void* b, int64_t E, int64_t N, int64_t K, void* out, hipStream_t stream);

// One wave: out[0] = shader-clock ticks, out[1] = 100 MHz ticks (>= ticks) of one sleep window.
hipError_t launch_clock_probe(unsigned long long* out, unsigned long long ticks, hipStream_t stream);

}  // namespace mxg
