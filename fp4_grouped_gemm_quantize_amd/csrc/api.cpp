// api.cpp -- the extern "C" entry points of libmxg.so: argument validation on
// the host (before anything is enqueued), then one launch per call.  No
// allocation, no host synchronisation, no state.
#include "mxg.h"
#include "mxg_internal.h"

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mxg_status from_hip(hipError_t e) { return e == hipSuccess ? MXG_SUCCESS : MXG_ERROR_LAUNCH; }

bool valid_fmt(int fmt) { return fmt == MXG_FP8_E4M3_ROWWISE || fmt == MXG_MXFP8_E4M3 || fmt == MXG_MXFP4_E2M1; }

// ---- MXG_VALIDATE: the optional check of the routing metadata (a debug mode).
thread_local char t_validation_msg[192] = "";

bool validation_on() {
    const char* v = getenv("MXG_VALIDATE");
    return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
}

// First violation in host copies of row_offsets [G + 1] and (if E > 0)
// expert_ids [G], written to `msg`; false if the routing is well formed.
bool find_violation(const uint32_t* off, const int32_t* ids, int64_t G, int64_t E, int64_t T, char* msg,
                    size_t len) {
    for (int64_t g = 0; g <= G; ++g) {
        if ((int64_t)off[g] > T) {
            snprintf(msg, len, "row_offsets[%lld] = %u exceeds total_rows = %lld", (long long)g, off[g],
                     (long long)T);
            return true;
        }
        if (g > 0 && off[g] < off[g - 1]) {
            snprintf(msg, len, "row_offsets[%lld] = %u is below row_offsets[%lld] = %u", (long long)g, off[g],
                     (long long)(g - 1), off[g - 1]);
            return true;
        }
    }
    if (ids != nullptr && E > 0)
        for (int64_t g = 0; g < G; ++g)
            if (ids[g] < 0 || ids[g] >= E) {
                snprintf(msg, len, "expert_ids[%lld] = %d lies outside [0, %lld)", (long long)g, ids[g],
                         (long long)E);
                return true;
            }
    return false;
}

// With MXG_VALIDATE set: copy the routing metadata to the host (synchronising
// `stream`) and refuse malformed routing before anything is launched.
// ids / E: the expert ids are checked when the entry point takes num_experts.
mxg_status check_routing(const uint32_t* off, const int32_t* ids, int64_t G, int64_t E, int64_t T,
                         hipStream_t stream) {
    if (!validation_on()) return MXG_SUCCESS;
    t_validation_msg[0] = '\0';
    std::vector<uint32_t> h_off((size_t)G + 1);
    std::vector<int32_t> h_ids(ids != nullptr && E > 0 ? (size_t)G : 0);
    if (hipMemcpyAsync(h_off.data(), off, sizeof(uint32_t) * h_off.size(), hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
        return MXG_ERROR_LAUNCH;
    if (!h_ids.empty() && hipMemcpyAsync(h_ids.data(), ids, sizeof(int32_t) * h_ids.size(), hipMemcpyDeviceToHost,
                                         stream) != hipSuccess)
        return MXG_ERROR_LAUNCH;
    if (hipStreamSynchronize(stream) != hipSuccess) return MXG_ERROR_LAUNCH;
    if (find_violation(h_off.data(), h_ids.empty() ? nullptr : h_ids.data(), G, E, T, t_validation_msg,
                       sizeof t_validation_msg))
        return MXG_ERROR_INVALID_VALUE;
    return MXG_SUCCESS;
}

mxg_status launch_gemm_checked(const mxg::GemmProblem& p, hipStream_t stream) {
    const mxg_status st = check_routing(p.off, p.ids, p.G, p.E, p.T, stream);
    if (st != MXG_SUCCESS) return st;
    return from_hip(mxg::launch_grouped_gemm(p, stream));
}

}  // namespace

extern "C" {

mxg_status mxg_clock_probe(unsigned long long* out, int64_t window_us, hipStream_t stream) {
    if (!out || !aligned(out, 8)) return MXG_ERROR_INVALID_VALUE;
    if (window_us <= 0 || window_us > MXG_CLOCK_PROBE_MAX_US) return MXG_ERROR_INVALID_VALUE;
    return from_hip(mxg::launch_clock_probe(out, (unsigned long long)window_us * 100ull, stream));
}

const char* mxg_validation_message(void) { return t_validation_msg; }

int mxg_routing_violation(const uint32_t* row_offsets_host, const int32_t* expert_ids_host, int32_t num_groups,
                          int32_t num_experts, int64_t total_rows, char* msg, int64_t msg_len) {
    if (!row_offsets_host || num_groups < 0 || total_rows < 0) return -1;
    char local[192];
    const bool bad = find_violation(row_offsets_host, expert_ids_host, num_groups, num_experts, total_rows, local,
                                    sizeof local);
    if (msg != nullptr && msg_len > 0) snprintf(msg, (size_t)msg_len, "%s", bad ? local : "");
    return bad ? 1 : 0;
}

const char* mxg_status_string(mxg_status status) {
    switch (status) {
        case MXG_SUCCESS:
            return "MXG_SUCCESS";
        case MXG_ERROR_INVALID_VALUE:
            return "MXG_ERROR_INVALID_VALUE: null pointer, bad enum, bad size or misaligned pointer";
        case MXG_ERROR_NOT_SUPPORTED:
            return "MXG_ERROR_NOT_SUPPORTED: K or I not a multiple of 32, too many groups, or format not offered";
        case MXG_ERROR_LAUNCH:
            return "MXG_ERROR_LAUNCH: the HIP runtime rejected a kernel launch";
    }
    return "unknown mxg_status";
}

mxg_status mx_grouped_quantize(mxg_format fmt, const void* x_bf16, void* q, void* scales,
                               const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                               int64_t total_rows, int64_t K, hipStream_t stream) {
    (void)expert_ids;  // not read by these formats (no per-expert tensor scale)
    if (!valid_fmt(fmt)) return MXG_ERROR_INVALID_VALUE;
    if (K <= 0 || total_rows < 0 || num_groups < 0) return MXG_ERROR_INVALID_VALUE;
    if (K % 32 != 0 || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!x_bf16 || !q || !scales || !row_offsets) return MXG_ERROR_INVALID_VALUE;
    if (!aligned(x_bf16, 16) || !aligned(q, 16) || (fmt == MXG_FP8_E4M3_ROWWISE && !aligned(scales, 4)) ||
        !aligned(row_offsets, 4))
        return MXG_ERROR_INVALID_VALUE;
    if (mxg_status st = check_routing(row_offsets, nullptr, num_groups, 0, total_rows, stream)) return st;
    return from_hip(mxg::launch_quantize((int)fmt, x_bf16, q, scales, row_offsets, num_groups, total_rows, K,
                                         stream));
}

mxg_status mx_grouped_quantize_gather(mxg_format fmt, const void* x_bf16, int64_t num_src_rows,
                                      const int32_t* indices, int32_t indices_divisor, void* q, void* scales,
                                      const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                      int64_t total_rows, int64_t K, hipStream_t stream) {
    (void)expert_ids;  // not read, as in mx_grouped_quantize
    if (!valid_fmt(fmt)) return MXG_ERROR_INVALID_VALUE;
    if (K <= 0 || total_rows < 0 || num_groups < 0 || num_src_rows < 0 || indices_divisor < 1)
        return MXG_ERROR_INVALID_VALUE;
    if (K % 32 != 0 || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!indices || !q || !scales || !row_offsets || (num_src_rows > 0 && !x_bf16)) return MXG_ERROR_INVALID_VALUE;
    if (!aligned(x_bf16, 16) || !aligned(q, 16) || (fmt == MXG_FP8_E4M3_ROWWISE && !aligned(scales, 4)) ||
        !aligned(row_offsets, 4) || !aligned(indices, 4))
        return MXG_ERROR_INVALID_VALUE;
    if (mxg_status st = check_routing(row_offsets, nullptr, num_groups, 0, total_rows, stream)) return st;
    return from_hip(mxg::launch_quantize_gather((int)fmt, x_bf16, num_src_rows, indices, indices_divisor, q, scales,
                                                row_offsets, num_groups, total_rows, K, stream));
}

mxg_status mx_grouped_quantize_scatter(mxg_format fmt, const void* x_tokens, int64_t num_tokens,
                                       const int32_t* row_of_slot, int32_t top_k, void* q, void* scales,
                                       const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                       int64_t total_rows, int64_t K, hipStream_t stream) {
    (void)expert_ids;  // not read, as in mx_grouped_quantize
    if (!valid_fmt(fmt)) return MXG_ERROR_INVALID_VALUE;
    if (K <= 0 || total_rows < 0 || num_groups < 0 || num_tokens < 0 || top_k < 1) return MXG_ERROR_INVALID_VALUE;
    if (K % 32 != 0 || num_groups > MXG_MAX_GROUPS || top_k > 64) return MXG_ERROR_NOT_SUPPORTED;
    if (fmt == MXG_FP8_E4M3_ROWWISE && K > 8192) return MXG_ERROR_NOT_SUPPORTED;
    if (num_tokens > INT32_MAX / top_k) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0 || num_tokens == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!x_tokens || !row_of_slot || !q || !scales || !row_offsets) return MXG_ERROR_INVALID_VALUE;
    if (!aligned(x_tokens, 16) || !aligned(q, 16) || (fmt == MXG_FP8_E4M3_ROWWISE && !aligned(scales, 4)) ||
        !aligned(row_offsets, 4) || !aligned(row_of_slot, 4))
        return MXG_ERROR_INVALID_VALUE;
    if (mxg_status st = check_routing(row_offsets, nullptr, num_groups, 0, total_rows, stream)) return st;
    return from_hip(mxg::launch_quantize_scatter((int)fmt, x_tokens, num_tokens, row_of_slot, top_k, q, scales,
                                                 row_offsets, num_groups, total_rows, K, stream));
}

mxg_status mx_grouped_quantize_nvfp4(const void* x_bf16, void* q, void* scales, const float* tensor_scales,
                                     const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                     int32_t num_experts, int64_t total_rows, int64_t K, hipStream_t stream) {
    if (K <= 0 || total_rows < 0 || num_groups < 0 || num_experts <= 0) return MXG_ERROR_INVALID_VALUE;
    if (K % 16 != 0 || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!x_bf16 || !q || !scales || !tensor_scales || !row_offsets || !expert_ids) return MXG_ERROR_INVALID_VALUE;
    if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(tensor_scales, 4) || !aligned(row_offsets, 4) ||
        !aligned(expert_ids, 4))
        return MXG_ERROR_INVALID_VALUE;
    if (mxg_status st = check_routing(row_offsets, expert_ids, num_groups, num_experts, total_rows, stream)) return st;
    return from_hip(mxg::launch_quantize_nvfp4(x_bf16, q, scales, tensor_scales, row_offsets, expert_ids, num_groups,
                                               num_experts, total_rows, K, stream));
}

mxg_status mx_grouped_quantize_padded(mxg_format fmt, const void* x_bf16, void* q, void* scales,
                                      const uint32_t* scales_offsets, int64_t scale_rows,
                                      const uint32_t* row_offsets, int32_t num_groups, int64_t total_rows, int64_t K,
                                      hipStream_t stream) {
    if (!valid_fmt(fmt)) return MXG_ERROR_INVALID_VALUE;
    if (K <= 0 || total_rows < 0 || num_groups < 0 || scale_rows < 0) return MXG_ERROR_INVALID_VALUE;
    if (fmt == MXG_FP8_E4M3_ROWWISE || K % 32 != 0 || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!x_bf16 || !q || !scales || !scales_offsets || !row_offsets) return MXG_ERROR_INVALID_VALUE;
    if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(scales_offsets, 4) || !aligned(row_offsets, 4))
        return MXG_ERROR_INVALID_VALUE;
    if (mxg_status st = check_routing(row_offsets, nullptr, num_groups, 0, total_rows, stream)) return st;
    return from_hip(mxg::launch_quantize_padded((int)fmt, x_bf16, q, scales, scales_offsets, scale_rows, row_offsets,
                                                num_groups, total_rows, K, stream));
}

mxg_status mx_grouped_quantize_nvfp4_padded(const void* x_bf16, void* q, void* scales, const float* tensor_scales,
                                            const uint32_t* scales_offsets, int64_t scale_rows,
                                            const uint32_t* row_offsets, const int32_t* expert_ids,
                                            int32_t num_groups, int32_t num_experts, int64_t total_rows, int64_t K,
                                            hipStream_t stream) {
    if (K <= 0 || total_rows < 0 || num_groups < 0 || num_experts <= 0 || scale_rows < 0)
        return MXG_ERROR_INVALID_VALUE;
    if (K % 16 != 0 || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!x_bf16 || !q || !scales || !tensor_scales || !scales_offsets || !row_offsets || !expert_ids)
        return MXG_ERROR_INVALID_VALUE;
    if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(tensor_scales, 4) || !aligned(scales_offsets, 4) ||
        !aligned(row_offsets, 4) || !aligned(expert_ids, 4))
        return MXG_ERROR_INVALID_VALUE;
    if (mxg_status st = check_routing(row_offsets, expert_ids, num_groups, num_experts, total_rows, stream)) return st;
    return from_hip(mxg::launch_quantize_nvfp4_padded(x_bf16, q, scales, tensor_scales, scales_offsets, scale_rows,
                                                      row_offsets, expert_ids, num_groups, num_experts, total_rows,
                                                      K, stream));
}

mxg_status mx_moe_combine(const void* y_bf16, int64_t total_rows, int64_t H, const int32_t* row_of_slot,
                          const float* weights, int64_t num_tokens, int32_t top_k, void* out_bf16,
                          hipStream_t stream) {
    if (H <= 0 || total_rows < 0 || num_tokens < 0 || top_k < 1) return MXG_ERROR_INVALID_VALUE;
    if (H % 8 != 0 || (int64_t)top_k * num_tokens > INT32_MAX) return MXG_ERROR_NOT_SUPPORTED;
    if (num_tokens == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!row_of_slot || !weights || !out_bf16 || (total_rows > 0 && !y_bf16)) return MXG_ERROR_INVALID_VALUE;
    if (!aligned(y_bf16, 16) || !aligned(out_bf16, 16) || !aligned(row_of_slot, 4) || !aligned(weights, 4))
        return MXG_ERROR_INVALID_VALUE;
    return from_hip(mxg::launch_combine(y_bf16, total_rows, H, row_of_slot, weights, num_tokens, top_k, out_bf16,
                                        stream));
}

static mxg_status check_gemm_common(mxg_format fmt, const void* a_q, const void* a_scales, const void* b_q,
                                    const void* b_scales, const uint32_t* row_offsets, const int32_t* expert_ids,
                                    int32_t num_groups, int32_t num_experts, int64_t total_rows, int64_t N,
                                    int64_t K) {
    if (!valid_fmt(fmt)) return MXG_ERROR_INVALID_VALUE;
    if (K <= 0 || N <= 0 || num_experts <= 0 || total_rows < 0 || num_groups < 0) return MXG_ERROR_INVALID_VALUE;
    if (K % 32 != 0 || K > MXG_MAX_K || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (N > INT32_MAX / 2 || total_rows > INT32_MAX) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // checked again by the caller: no-op
    if (!a_q || !a_scales || !b_q || !b_scales || !row_offsets || !expert_ids) return MXG_ERROR_INVALID_VALUE;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(row_offsets, 4) || !aligned(expert_ids, 4))
        return MXG_ERROR_INVALID_VALUE;
    if (fmt == MXG_FP8_E4M3_ROWWISE && (!aligned(a_scales, 4) || !aligned(b_scales, 4)))
        return MXG_ERROR_INVALID_VALUE;
    // block scales: 16-byte direct-to-LDS chunks when K is a multiple of 1024
    if (fmt != MXG_FP8_E4M3_ROWWISE && (!aligned(a_scales, 16) || !aligned(b_scales, 16)))
        return MXG_ERROR_INVALID_VALUE;
    return MXG_SUCCESS;
}

mxg_status mx_grouped_matmul(mxg_format fmt, const void* a_q, const void* a_scales, const void* b_q,
                             const void* b_scales, void* c_bf16, const uint32_t* row_offsets,
                             const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                             int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                             hipStream_t stream) {
    mxg_status st = check_gemm_common(fmt, a_q, a_scales, b_q, b_scales, row_offsets, expert_ids, num_groups,
                                      num_experts, total_rows, N, K);
    if (st != MXG_SUCCESS) return st;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;
    if (!c_bf16 || !aligned(c_bf16, 16)) return MXG_ERROR_INVALID_VALUE;
    mxg::GemmProblem p{(int)fmt, a_q, a_scales, b_q, b_scales, c_bf16, nullptr, nullptr, row_offsets, expert_ids,
                       num_groups, num_experts, total_rows, N, K, max_rows_per_group_hint};
    return launch_gemm_checked(p, stream);
}

int32_t mxg_fp8_tile(int32_t num_groups, int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                     int32_t prepared) {
    if (num_groups <= 0 || total_rows <= 0 || N <= 0 || K <= 0) return 0;
    if (K % 32 != 0 || K > MXG_MAX_K || num_groups > MXG_MAX_GROUPS || N > INT32_MAX / 2 || total_rows > INT32_MAX)
        return 0;
    mxg::GemmProblem p{};
    p.fmt = MXG_FP8_E4M3_ROWWISE;
    p.G = num_groups;
    p.T = total_rows;
    p.N = N;
    p.K = K;
    p.max_rows_hint = max_rows_per_group_hint;
    p.b_prepared = prepared != 0;
    return mxg::fp8_tile_choice(p);
}

// E * ceil(N / 256) * 256 * K fits in int64
static bool prepared_size_fits(int64_t num_experts, int64_t N, int64_t K) {
    const int64_t rows = (N + 255) / 256 * 256;
    return rows <= INT64_MAX / num_experts && rows * num_experts <= INT64_MAX / K;
}

int64_t mx_prepared_weights_bytes(int64_t num_experts, int64_t N, int64_t K) {
    if (num_experts <= 0 || N <= 0 || K <= 0 || K % 64 != 0) return -1;
    if (N > INT32_MAX / 2 || K > INT32_MAX / 2 || !prepared_size_fits(num_experts, N, K)) return -1;
    return mxg::prepared_weights_bytes(num_experts, N, K);
}

mxg_status mx_prepare_weights_fp8(const void* b_q, int32_t num_experts, int64_t N, int64_t K, void* b_prepared,
                                  hipStream_t stream) {
    if (num_experts <= 0 || N <= 0 || K <= 0) return MXG_ERROR_INVALID_VALUE;
    if (K % 64 != 0 || N > INT32_MAX / 2 || K > INT32_MAX / 2 || !prepared_size_fits(num_experts, N, K))
        return MXG_ERROR_NOT_SUPPORTED;
    if (!b_q || !b_prepared || !aligned(b_q, 16) || !aligned(b_prepared, 16)) return MXG_ERROR_INVALID_VALUE;
    return from_hip(mxg::launch_prepare_weights(b_q, num_experts, N, K, b_prepared, stream));
}

mxg_status mx_grouped_matmul_prepared(const void* a_q, const void* a_scales, const void* b_prepared,
                                      const void* b_scales, void* c_bf16, const uint32_t* row_offsets,
                                      const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                                      int64_t total_rows, int64_t N, int64_t K, hipStream_t stream) {
    mxg_status st = check_gemm_common(MXG_FP8_E4M3_ROWWISE, a_q, a_scales, b_prepared, b_scales, row_offsets,
                                      expert_ids, num_groups, num_experts, total_rows, N, K);
    if (st != MXG_SUCCESS) return st;
    if (K % 64 != 0) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;
    if (!c_bf16 || !aligned(c_bf16, 16)) return MXG_ERROR_INVALID_VALUE;
    mxg::GemmProblem p{0, a_q, a_scales, b_prepared, b_scales, c_bf16, nullptr, nullptr, row_offsets, expert_ids,
                       num_groups, num_experts, total_rows, N, K, 0};
    p.b_prepared = true;
    return launch_gemm_checked(p, stream);
}

mxg_status mx_grouped_matmul_nvfp4(const void* a_q, const void* a_scales, const void* b_q, const void* b_scales,
                                   const float* expert_scales, void* c_bf16, const uint32_t* row_offsets,
                                   const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                                   int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                                   hipStream_t stream) {
    if (K <= 0 || N <= 0 || num_experts <= 0 || total_rows < 0 || num_groups < 0) return MXG_ERROR_INVALID_VALUE;
    if (K % 512 != 0 || K > MXG_MAX_K || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (N > INT32_MAX / 2 || total_rows > INT32_MAX) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!a_q || !a_scales || !b_q || !b_scales || !expert_scales || !c_bf16 || !row_offsets || !expert_ids)
        return MXG_ERROR_INVALID_VALUE;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_scales, 16) || !aligned(b_scales, 16) ||
        !aligned(c_bf16, 16) || !aligned(expert_scales, 4) || !aligned(row_offsets, 4) || !aligned(expert_ids, 4))
        return MXG_ERROR_INVALID_VALUE;
    mxg::GemmProblem p{3, a_q, a_scales, b_q, b_scales, c_bf16, nullptr, nullptr, row_offsets, expert_ids,
                       num_groups, num_experts, total_rows, N, K, max_rows_per_group_hint, expert_scales};
    return launch_gemm_checked(p, stream);
}

mxg_status mx_grouped_matmul_nvfp4_padded(const void* a_q, const void* a_scales, const uint32_t* a_scales_offsets,
                                          int64_t a_scale_rows, const void* b_q, const void* b_scales,
                                          const float* expert_scales, void* c_bf16, const uint32_t* row_offsets,
                                          const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                                          int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                                          hipStream_t stream) {
    if (K <= 0 || N <= 0 || num_experts <= 0 || total_rows < 0 || num_groups < 0 || a_scale_rows < 0)
        return MXG_ERROR_INVALID_VALUE;
    if (K % 512 != 0 || K > MXG_MAX_K || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (N > INT32_MAX / 2 || total_rows > INT32_MAX) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!a_q || !a_scales || !a_scales_offsets || !b_q || !b_scales || !expert_scales || !c_bf16 || !row_offsets ||
        !expert_ids)
        return MXG_ERROR_INVALID_VALUE;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || !aligned(a_scales, 16) || !aligned(b_scales, 16) ||
        !aligned(c_bf16, 16) || !aligned(expert_scales, 4) || !aligned(a_scales_offsets, 4) ||
        !aligned(row_offsets, 4) || !aligned(expert_ids, 4))
        return MXG_ERROR_INVALID_VALUE;
    mxg::GemmProblem p{3, a_q, a_scales, b_q, b_scales, c_bf16, nullptr, nullptr, row_offsets, expert_ids,
                       num_groups, num_experts, total_rows, N, K, max_rows_per_group_hint, expert_scales, nullptr,
                       nullptr, a_scales_offsets, a_scale_rows};
    return launch_gemm_checked(p, stream);
}

// Padded A scales: the MX GEMM / fused GEMM with a_scales in the layout of
// mx_grouped_quantize_padded.
static mxg_status check_padded(mxg_format fmt, const uint32_t* a_scales_offsets, int64_t a_scale_rows,
                               const void* a_scales) {
    if (a_scale_rows < 0) return MXG_ERROR_INVALID_VALUE;
    if (fmt == MXG_FP8_E4M3_ROWWISE) return MXG_ERROR_NOT_SUPPORTED;
    if (!a_scales_offsets || !aligned(a_scales_offsets, 4) || !aligned(a_scales, 16)) return MXG_ERROR_INVALID_VALUE;
    return MXG_SUCCESS;
}

mxg_status mx_grouped_matmul_padded(mxg_format fmt, const void* a_q, const void* a_scales,
                                    const uint32_t* a_scales_offsets, int64_t a_scale_rows, const void* b_q,
                                    const void* b_scales, void* c_bf16, const uint32_t* row_offsets,
                                    const int32_t* expert_ids, int32_t num_groups, int32_t num_experts,
                                    int64_t total_rows, int64_t N, int64_t K, int64_t max_rows_per_group_hint,
                                    hipStream_t stream) {
    mxg_status st = check_gemm_common(fmt, a_q, a_scales, b_q, b_scales, row_offsets, expert_ids, num_groups,
                                      num_experts, total_rows, N, K);
    if (st != MXG_SUCCESS) return st;
    if (a_scale_rows < 0) return MXG_ERROR_INVALID_VALUE;
    if (fmt == MXG_FP8_E4M3_ROWWISE) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;
    if ((st = check_padded(fmt, a_scales_offsets, a_scale_rows, a_scales)) != MXG_SUCCESS) return st;
    if (!c_bf16 || !aligned(c_bf16, 16)) return MXG_ERROR_INVALID_VALUE;
    mxg::GemmProblem p{(int)fmt, a_q, a_scales, b_q, b_scales, c_bf16, nullptr, nullptr, row_offsets, expert_ids,
                       num_groups, num_experts, total_rows, N, K, max_rows_per_group_hint, nullptr, nullptr, nullptr,
                       a_scales_offsets, a_scale_rows};
    return launch_gemm_checked(p, stream);
}

mxg_status mx_grouped_matmul_swiglu_padded(mxg_format fmt, const void* a_q, const void* a_scales,
                                           const uint32_t* a_scales_offsets, int64_t a_scale_rows, const void* w_q,
                                           const void* w_scales, void* y_q, void* y_scales,
                                           const uint32_t* row_offsets, const int32_t* expert_ids,
                                           int32_t num_groups, int32_t num_experts, int64_t total_rows, int64_t I,
                                           int64_t K, int64_t max_rows_per_group_hint, hipStream_t stream) {
    if (I <= 0) return MXG_ERROR_INVALID_VALUE;
    mxg_status st = check_gemm_common(fmt, a_q, a_scales, w_q, w_scales, row_offsets, expert_ids, num_groups,
                                      num_experts, total_rows, 2 * I, K);
    if (st != MXG_SUCCESS) return st;
    if (a_scale_rows < 0) return MXG_ERROR_INVALID_VALUE;
    if (fmt == MXG_FP8_E4M3_ROWWISE || I % 32 != 0) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;
    if ((st = check_padded(fmt, a_scales_offsets, a_scale_rows, a_scales)) != MXG_SUCCESS) return st;
    if (!y_q || !y_scales || !aligned(y_q, 16)) return MXG_ERROR_INVALID_VALUE;
    mxg::GemmProblem p{(int)fmt, a_q, a_scales, w_q, w_scales, nullptr, y_q, y_scales, row_offsets, expert_ids,
                       num_groups, num_experts, total_rows, 2 * I, K, max_rows_per_group_hint, nullptr, nullptr,
                       nullptr, a_scales_offsets, a_scale_rows};
    return launch_gemm_checked(p, stream);
}

mxg_status mx_grouped_matmul_swiglu_nvfp4(const void* a_q, const void* a_scales, const void* w_q,
                                          const void* w_scales, const float* expert_scales,
                                          const void* a_row_scales_bf16, const float* y_tensor_scales, void* y_q,
                                          void* y_scales, const uint32_t* row_offsets, const int32_t* expert_ids,
                                          int32_t num_groups, int32_t num_experts, int64_t total_rows, int64_t I,
                                          int64_t K, int64_t max_rows_per_group_hint, hipStream_t stream) {
    if (K <= 0 || I <= 0 || num_experts <= 0 || total_rows < 0 || num_groups < 0) return MXG_ERROR_INVALID_VALUE;
    if (K % 512 != 0 || K > MXG_MAX_K || I % 32 != 0 || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (I > INT32_MAX / 4 || total_rows > INT32_MAX) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;  // nothing is read or written
    if (!a_q || !a_scales || !w_q || !w_scales || !expert_scales || !y_tensor_scales || !y_q || !y_scales ||
        !row_offsets || !expert_ids)
        return MXG_ERROR_INVALID_VALUE;
    if (!aligned(a_q, 16) || !aligned(a_scales, 16) || !aligned(w_q, 16) || !aligned(w_scales, 16) ||
        !aligned(y_q, 16) || !aligned(expert_scales, 4) || !aligned(y_tensor_scales, 4) ||
        !aligned(a_row_scales_bf16, 2) || !aligned(row_offsets, 4) || !aligned(expert_ids, 4))
        return MXG_ERROR_INVALID_VALUE;
    mxg::GemmProblem p{3, a_q, a_scales, w_q, w_scales, nullptr, y_q, y_scales, row_offsets, expert_ids,
                       num_groups, num_experts, total_rows, 2 * I, K, max_rows_per_group_hint, expert_scales,
                       a_row_scales_bf16, y_tensor_scales};
    return launch_gemm_checked(p, stream);
}

mxg_status mx_silu_quantize_nvfp4(const void* h_bf16, void* y_q, void* y_scales, const float* y_tensor_scales,
                                  const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                  int32_t num_experts, int64_t total_rows, int64_t I, hipStream_t stream) {
    if (I <= 0 || total_rows < 0 || num_groups < 0 || num_experts <= 0) return MXG_ERROR_INVALID_VALUE;
    if (I % 16 != 0 || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;
    if (!h_bf16 || !y_q || !y_scales || !y_tensor_scales || !row_offsets || !expert_ids)
        return MXG_ERROR_INVALID_VALUE;
    if (!aligned(h_bf16, 16) || !aligned(y_q, 16) || !aligned(y_tensor_scales, 4) || !aligned(row_offsets, 4) ||
        !aligned(expert_ids, 4))
        return MXG_ERROR_INVALID_VALUE;
    if (mxg_status st = check_routing(row_offsets, expert_ids, num_groups, num_experts, total_rows, stream)) return st;
    return from_hip(mxg::launch_silu_quantize_nvfp4(h_bf16, y_q, y_scales, y_tensor_scales, row_offsets, expert_ids,
                                                    num_groups, num_experts, total_rows, I, stream));
}

mxg_status mx_grouped_matmul_swiglu(mxg_format fmt, const void* a_q, const void* a_scales, const void* w_q,
                                    const void* w_scales, void* y_q, void* y_scales,
                                    const uint32_t* row_offsets, const int32_t* expert_ids, int32_t num_groups,
                                    int32_t num_experts, int64_t total_rows, int64_t I, int64_t K,
                                    int64_t max_rows_per_group_hint, hipStream_t stream) {
    if (I <= 0) return MXG_ERROR_INVALID_VALUE;
    mxg_status st = check_gemm_common(fmt, a_q, a_scales, w_q, w_scales, row_offsets, expert_ids, num_groups,
                                      num_experts, total_rows, 2 * I, K);
    if (st != MXG_SUCCESS) return st;
    if (fmt == MXG_FP8_E4M3_ROWWISE || I % 32 != 0) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;
    if (!y_q || !y_scales || !aligned(y_q, 16)) return MXG_ERROR_INVALID_VALUE;
    mxg::GemmProblem p{(int)fmt, a_q, a_scales, w_q, w_scales, nullptr, y_q, y_scales, row_offsets, expert_ids,
                       num_groups, num_experts, total_rows, 2 * I, K, max_rows_per_group_hint};
    return launch_gemm_checked(p, stream);
}

mxg_status mx_silu_quantize(const void* h_bf16, void* y_q, void* y_scales, const uint32_t* row_offsets,
                            int32_t num_groups, int64_t total_rows, int64_t I, hipStream_t stream) {
    if (I <= 0 || total_rows < 0 || num_groups < 0) return MXG_ERROR_INVALID_VALUE;
    if (I % 32 != 0 || num_groups > MXG_MAX_GROUPS) return MXG_ERROR_NOT_SUPPORTED;
    if (total_rows == 0 || num_groups == 0) return MXG_SUCCESS;
    if (!h_bf16 || !y_q || !y_scales || !row_offsets) return MXG_ERROR_INVALID_VALUE;
    if (!aligned(h_bf16, 16) || !aligned(y_q, 16) || !aligned(row_offsets, 4)) return MXG_ERROR_INVALID_VALUE;
    if (mxg_status st = check_routing(row_offsets, nullptr, num_groups, 0, total_rows, stream)) return st;
    return from_hip(mxg::launch_silu_quantize(h_bf16, y_q, y_scales, row_offsets, num_groups, total_rows, I, stream));
}

}  // extern "C"
