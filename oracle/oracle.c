/*
 * oracle.c -- plain, slow CPU reference for the ragged MoE expert path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle: only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * source, header, table or helper with the GPU library, and it never calls it.
 *
 * What it follows (pages cited by title and section):
 *   - grouped_matmul_rowwise_dynamic_scaled_fp8, description: each routed row
 *     t of group g and each column n of the output take
 *       out[t,n] = (sum_k a[t,k] * b[expert_ids[g],n,k]) * a_scale[t] * b_scale[expert_ids[g],n]
 *     with weights [num_experts, N, K] (K innermost), row offsets uint32
 *     [num_groups+1], expert ids int32 [num_groups], bf16 output.
 *   - grouped_quantize_dynamic_scaled_fp4_async_kernel, description: per-expert
 *     dynamic quantization of BF16 activations to MXFP4 / MXFP8 block formats.
 *   - NvMxf4f8Strategy, grouped_quantize() / quantize(): (q, scales) pairs with a
 *     group_size; grouped_matmul(): block-scaled grouped matmul;
 *     fused_silu_quantize(): gated activation then quantization;
 *     grouped_matmul_swiglu(): the same two steps fused, byte-identical.
 *   - Struct_ep_dispatch_mxfp4, execute: MX activation scales are E8M0 and one
 *     scale covers a K block (K_SCALES per row).
 *   - NvMxf4f8Strategy, is_nvfp4 / grouped_quantize(input_scale) /
 *     grouped_matmul(expert_scales) and the kernel's sf_tensor: the NVFP4
 *     variant (readings at its functions below).
 *   - Element and scale encodings follow the public OCP 8-bit floating point
 *     (OFP8, "E4M3" with no infinities) and OCP Microscaling v1.0 (E2M1, E8M0,
 *     32-element blocks, shared exponent = floor(log2 amax) - emax_elem)
 *     specifications.
 *
 * Readings where the pages are silent (rounding is round-to-nearest-even,
 * overflow saturates to the largest finite code, a zero row or block gets a
 * zero scale, the fp8 rowwise scale is amax/448 and the element is
 * fl32(x / scale), gate/up rows are interleaved 2j / 2j+1, silu(z) =
 * z / (1 + e^-z), g, u and y are rounded to bf16) are listed with the
 * repository's design notes.
 *
 * All arithmetic that decides a value is fp64 except where a reading fixes fp32
 * (the rowwise scale and quotient).  Every loop is the definition written out;
 * OpenMP only spreads independent rows over threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Status codes of this oracle (not the GPU library's).                        */
#define MXO_OK 0
#define MXO_EINVAL 1

/* Element formats. */
#define MXO_E4M3 0
#define MXO_E2M1 1

int mxo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Decoders: closed forms of each code (OFP8 E4M3 "fn", OCP MX E2M1, E8M0).     */

/* bf16 is the top half of an IEEE binary32. */
double mxo_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E4M3 "fn": sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities. */
double mxo_e4m3_value(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = (double)m * ldexp(1.0, -9);
    else
        v = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
    return s ? -v : v;
}

/* E2M1 (low nibble): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent 0 is subnormal (m * 0.5).  Values 0, .5, 1, 1.5, 2, 3, 4, 6. */
double mxo_e2m1_value(uint8_t code) {
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 0x3;
    int m = code & 0x1;
    double v;
    if (e == 0)
        v = (double)m * 0.5;
    else
        v = (1.0 + (double)m / 2.0) * ldexp(1.0, e - 1);
    return s ? -v : v;
}

/* E8M0 scale: 2^(c - 127); 0xFF is NaN. */
double mxo_e8m0_value(uint8_t code) {
    if (code == 0xFF) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* ------------------------------------------------------------------------- */
/* Encoders.  Input: any double.  Round to nearest, ties to even mantissa;     */
/* magnitudes at or beyond the largest finite code saturate to it; the sign   */
/* bit is always kept (so a negative value that rounds to zero is -0).        */

/* floor(log2(a)) for a > 0, exact (frexp gives a = f * 2^e, f in [0.5, 1)). */
static int floor_log2(double a) {
    int e;
    frexp(a, &e);
    return e - 1;
}

uint8_t mxo_e4m3_encode(double v) {
    uint8_t s = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (isnan(v)) return (uint8_t)(s | 0x7F);
    if (a >= 448.0) return (uint8_t)(s | 0x7E); /* saturate: max finite 1.75 * 2^8 */
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: value = m * 2^-9, m in 0..8 (m == 8 is the min normal 0x08) */
        double m = nearbyint(a * 512.0);
        return (uint8_t)(s | (uint8_t)m);
    }
    int e = floor_log2(a); /* -6 .. 8 */
    double m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8.0) {
        e += 1;
        m = 0.0;
    }
    return (uint8_t)(s | (uint8_t)((e + 7) << 3) | (uint8_t)m);
}

uint8_t mxo_e2m1_encode(double v) {
    uint8_t s = signbit(v) ? 0x8 : 0x0;
    double a = fabs(v);
    if (isnan(v)) return (uint8_t)(s | 0x7); /* no NaN code: out of contract */
    if (a >= 6.0) return (uint8_t)(s | 0x7); /* saturate: max finite 1.5 * 2^2 */
    if (a < 1.0) {
        /* subnormal range: value = m * 0.5, m in 0..2 (m == 2 is 1.0 = code 0x2) */
        double m = nearbyint(a * 2.0);
        return (uint8_t)(s | (uint8_t)m);
    }
    int e = floor_log2(a); /* 0 .. 2 */
    double m = nearbyint((ldexp(a, -e) - 1.0) * 2.0);
    if (m == 2.0) {
        e += 1;
        m = 0.0;
    }
    return (uint8_t)(s | (uint8_t)((e + 1) << 1) | (uint8_t)m);
}

/* Round a double straight to bf16 (8 significant bits), ties to even.  No
 * intermediate fp32 rounding, so there is no double rounding. */
uint16_t mxo_bf16_round(double v) {
    uint16_t s = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(s | 0x7FC0);
    if (a == 0.0) return s;
    if (isinf(v)) return (uint16_t)(s | 0x7F80);
    int e = floor_log2(a);
    if (e < -126) e = -126;          /* subnormal spacing is 2^-133 */
    double ulp = ldexp(1.0, e - 7);
    double q = nearbyint(a / ulp) * ulp;
    if (q >= ldexp(1.0, 128)) return (uint16_t)(s | 0x7F80); /* overflow to inf */
    float f = (float)q;              /* exact: q has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(s | (uint16_t)(u >> 16));
}

/* ------------------------------------------------------------------------- */
/* Group structure (grouped_matmul_rowwise_dynamic_scaled_fp8, Args: a_offsets
 * and expert_ids).  Group g covers rows [off[g], off[g+1]).  A group is taken
 * only when its start does not exceed its end; both ends are clamped to T.
 * These helpers are only used to decide which rows exist; no arithmetic.     */

static void group_range(const uint32_t* off, int32_t g, int64_t T, int64_t* lo, int64_t* hi) {
    int64_t a = (int64_t)off[g], b = (int64_t)off[g + 1];
    if (a > T) a = T;
    if (b > T) b = T;
    *lo = a;
    *hi = b;
}

/* The group that covers row t, or -1.  When several (malformed, overlapping)
 * groups cover t, -2.  A group with an expert id outside [0, E) is not taken
 * (pass E <= 0 to ignore ids). */
static int32_t group_of_row(const uint32_t* off, const int32_t* ids, int32_t G, int32_t E, int64_t T,
                            int64_t t) {
    int32_t found = -1;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        if (lo > hi) continue;
        if (E > 0 && (ids[g] < 0 || ids[g] >= E)) continue;
        if (t >= lo && t < hi) {
            if (found >= 0) return -2;
            found = g;
        }
    }
    return found;
}

int32_t mxo_group_of_row(const uint32_t* off, const int32_t* ids, int32_t G, int32_t E, int64_t T,
                         int64_t t) {
    return group_of_row(off, ids, G, E, T, t);
}

/* ------------------------------------------------------------------------- */
/* Quantize (grouped_quantize_dynamic_scaled_fp4_async_kernel; NvMxf4f8Strategy
 * grouped_quantize()).  Every row covered by a group is quantized; other rows
 * of q and scales are left as they were.                                     */

/* FP8 rowwise, one row: scale = fl32(amax / 448), element = enc(fl32(x / scale)).
 * (grouped_matmul_rowwise_dynamic_scaled_fp8: per-token activation scales.) */
static void quantize_row_fp8(const uint16_t* x, int64_t K, uint8_t* q, float* scale) {
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = fabsf((float)mxo_bf16_value(x[k]));
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale = 0.0f;
        for (int64_t k = 0; k < K; ++k) q[k] = (x[k] & 0x8000) ? 0x80 : 0x00;
        return;
    }
    volatile float s = amax / 448.0f; /* IEEE binary32 division, round to nearest even */
    *scale = s;
    for (int64_t k = 0; k < K; ++k) {
        float xf = (float)mxo_bf16_value(x[k]);
        volatile float v = xf / s; /* IEEE binary32 division */
        q[k] = mxo_e4m3_encode((double)v);
    }
}

/* One MX block of n elements: shared exponent X = clamp(floor(log2 amax) -
 * emax_elem, -127, 127), scale code X + 127, elements enc(x * 2^-X) (exact). */
static uint8_t quantize_block_mx(int elem, const double* x, int n, uint8_t* codes) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    if (amax == 0.0) {
        for (int i = 0; i < n; ++i)
            codes[i] = signbit(x[i]) ? (elem == MXO_E4M3 ? 0x80 : 0x8) : 0x0;
        return 0x00;
    }
    int emax_elem = (elem == MXO_E4M3) ? 8 : 2;
    int X = floor_log2(amax) - emax_elem;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    for (int i = 0; i < n; ++i) {
        double v = ldexp(x[i], -X);
        codes[i] = (elem == MXO_E4M3) ? mxo_e4m3_encode(v) : mxo_e2m1_encode(v);
    }
    return (uint8_t)(X + 127);
}

/* MX one row of K bf16 values: codes (e4m3: K bytes; e2m1: K/2 bytes, element
 * 2i in the low nibble of byte i) and K/32 E8M0 scales. */
static void quantize_row_mx(int elem, const uint16_t* x, int64_t K, uint8_t* q, uint8_t* s) {
    double blk[32];
    uint8_t codes[32];
    for (int64_t b = 0; b < K / 32; ++b) {
        for (int i = 0; i < 32; ++i) blk[i] = mxo_bf16_value(x[b * 32 + i]);
        s[b] = quantize_block_mx(elem, blk, 32, codes);
        if (elem == MXO_E4M3) {
            for (int i = 0; i < 32; ++i) q[b * 32 + i] = codes[i];
        } else {
            for (int i = 0; i < 16; ++i)
                q[b * 16 + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    }
}

/* fmt: 0 = FP8 rowwise (scales fp32 [T]); 1 = MXFP8 (u8 [T, K/32]);
 * 2 = MXFP4 (codes [T, K/2], scales u8 [T, K/32]). */
int mxo_quantize(int fmt, const uint16_t* x, uint8_t* q, void* scales, const uint32_t* off, int32_t G,
                 int64_t T, int64_t K) {
    if (!x || !q || !scales || !off || G < 0 || T < 0 || K <= 0 || (K % 32) != 0) return MXO_EINVAL;
    if (fmt < 0 || fmt > 2) return MXO_EINVAL;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        if (lo > hi) continue;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t t = lo; t < hi; ++t) {
            if (fmt == 0) {
                quantize_row_fp8(x + t * K, K, q + t * K, (float*)scales + t);
            } else if (fmt == 1) {
                quantize_row_mx(MXO_E4M3, x + t * K, K, q + t * K, (uint8_t*)scales + t * (K / 32));
            } else {
                quantize_row_mx(MXO_E2M1, x + t * K, K, q + t * (K / 2), (uint8_t*)scales + t * (K / 32));
            }
        }
    }
    return MXO_OK;
}

/* Gathered grouped quantize (NvMxf4f8Strategy, grouped_quantize(): indices,
 * indices_divisor; the pages name the two parameters without defining them,
 * and the reading taken is: routed row t is source row idx[t] / div of x,
 * which has nsrc rows).  Row t of q / scales is what mxo_quantize writes for
 * that source row; a covered row whose index is negative or names no source
 * row is left untouched, as is every uncovered row.                        */
int mxo_quantize_gather(int fmt, const uint16_t* x, int64_t nsrc, const int32_t* idx, int32_t div, uint8_t* q,
                        void* scales, const uint32_t* off, int32_t G, int64_t T, int64_t K) {
    if (!q || !scales || !off || !idx || G < 0 || T < 0 || nsrc < 0 || div < 1 || K <= 0 || (K % 32) != 0)
        return MXO_EINVAL;
    if (nsrc > 0 && !x) return MXO_EINVAL;
    if (fmt < 0 || fmt > 2) return MXO_EINVAL;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        if (lo > hi) continue;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t t = lo; t < hi; ++t) {
            if (idx[t] < 0) continue;
            const int64_t src = (int64_t)idx[t] / div;
            if (src >= nsrc) continue;
            const uint16_t* xr = x + src * K;
            if (fmt == 0) {
                quantize_row_fp8(xr, K, q + t * K, (float*)scales + t);
            } else if (fmt == 1) {
                quantize_row_mx(MXO_E4M3, xr, K, q + t * K, (uint8_t*)scales + t * (K / 32));
            } else {
                quantize_row_mx(MXO_E2M1, xr, K, q + t * (K / 2), (uint8_t*)scales + t * (K / 32));
            }
        }
    }
    return MXO_OK;
}

/* Token-major form of the gathered quantize (NvMxf4f8Strategy,
 * grouped_quantize(), Args indices and indices_divisor, read through the
 * inverse slot map the combine uses).  For token s < ntok and slot k < top_k,
 * routed row r = ros[s * top_k + k] receives the quantization of token row s
 * when r lies in [0, T) and a group covers it; every other row of q and
 * scales is left as it was.  A routed row is a copy of its token's row, so
 * each token row is quantized once here and its result copied to the rows.  */
int mxo_quantize_scatter(int fmt, const uint16_t* x, int64_t ntok, const int32_t* ros, int32_t top_k, uint8_t* q,
                         void* scales, const uint32_t* off, int32_t G, int64_t T, int64_t K) {
    if (!q || !scales || !off || !ros || G < 0 || T < 0 || ntok < 0 || top_k < 1 || K <= 0 || (K % 32) != 0)
        return MXO_EINVAL;
    if (ntok > 0 && !x) return MXO_EINVAL;
    if (fmt < 0 || fmt > 2) return MXO_EINVAL;
    const int64_t qcols = fmt == 2 ? K / 2 : K;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t s = 0; s < ntok; ++s) {
        uint8_t* qt = (uint8_t*)malloc((size_t)qcols);
        const uint16_t* xr = x + s * K;
        uint8_t* sblk = (uint8_t*)malloc((size_t)(K / 32 > 4 ? K / 32 : 4));
        if (!qt || !sblk) {
            free(qt);
            free(sblk);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        float sf = 0.0f;
        if (fmt == 0) quantize_row_fp8(xr, K, qt, &sf);
        else quantize_row_mx(fmt == 1 ? MXO_E4M3 : MXO_E2M1, xr, K, qt, sblk);
        for (int32_t k = 0; k < top_k; ++k) {
            const int32_t r = ros[s * top_k + k];
            if (r < 0 || (int64_t)r >= T) continue;
            if (group_of_row(off, NULL, G, 0, T, r) == -1) continue;  /* not covered */
            memcpy(q + (int64_t)r * qcols, qt, (size_t)qcols);
            if (fmt == 0) ((float*)scales)[r] = sf;
            else memcpy((uint8_t*)scales + (int64_t)r * (K / 32), sblk, (size_t)(K / 32));
        }
        free(sblk);
        free(qt);
    }
    return failed ? MXO_EINVAL : MXO_OK;
}

/* ------------------------------------------------------------------------- */
/* Grouped GEMM on a list of rows (grouped_matmul_rowwise_dynamic_scaled_fp8,
 * description; NvMxf4f8Strategy grouped_matmul()).  For each listed row t the
 * full output row is computed: out[i, n] for i = position of t in `rows`.
 *   exact[i,n]  = the unrounded fp64 value,
 *   bound[i,n]  = sum_k |a * b| * scales (the tolerance's reference scale),
 *   out[i,n]    = bf16 round-to-nearest-even of exact,
 *   group[i]    = covering group, -1 if none (row left out), -2 if ambiguous.
 * Any of exact / bound / out may be NULL.                                    */

static double dec_elem(int elem, const uint8_t* row, int64_t k) {
    if (elem == MXO_E4M3) return mxo_e4m3_value(row[k]);
    uint8_t byte = row[k / 2];
    return mxo_e2m1_value((k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF));
}

/* fmt: 0 = FP8 rowwise (a_scale fp32 [T], b_scale fp32 [E, N]);
 *      1 = MXFP8, 2 = MXFP4 (a_scale u8 [T, K/32], b_scale u8 [E, N, K/32]). */
int mxo_gemm_rows(int fmt, const uint8_t* a, const void* a_scale, const uint8_t* b, const void* b_scale,
                  const uint32_t* off, const int32_t* ids, int32_t G, int32_t E, int64_t T, int64_t N,
                  int64_t K, const int64_t* rows, int64_t nrows, uint16_t* out, double* exact, double* bound,
                  int32_t* group) {
    if (!a || !a_scale || !b || !b_scale || !off || !ids || !rows) return MXO_EINVAL;
    if (fmt < 0 || fmt > 2 || G < 0 || E <= 0 || T < 0 || N <= 0 || K <= 0 || (K % 32) != 0) return MXO_EINVAL;
    int elem = (fmt == 2) ? MXO_E2M1 : MXO_E4M3;
    int64_t row_bytes = (fmt == 2) ? K / 2 : K;
    int64_t nblk = K / 32;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t t = rows[i];
        int32_t g = (t >= 0 && t < T) ? group_of_row(off, ids, G, E, T, t) : -1;
        if (group) group[i] = g;
        if (g < 0) continue;
        int32_t e = ids[g];
        const uint8_t* arow = a + t * row_bytes;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* brow = b + ((int64_t)e * N + n) * row_bytes;
            double acc = 0.0, mag = 0.0;
            if (fmt == 0) {
                double sa = (double)((const float*)a_scale)[t];
                double sb = (double)((const float*)b_scale)[(int64_t)e * N + n];
                for (int64_t k = 0; k < K; ++k) {
                    double p = dec_elem(elem, arow, k) * dec_elem(elem, brow, k);
                    acc += p;
                    mag += fabs(p);
                }
                acc = acc * sa * sb;
                mag = mag * fabs(sa) * fabs(sb);
            } else {
                const uint8_t* sa = (const uint8_t*)a_scale + t * nblk;
                const uint8_t* sb = (const uint8_t*)b_scale + ((int64_t)e * N + n) * nblk;
                for (int64_t blk = 0; blk < nblk; ++blk) {
                    double part = 0.0, pmag = 0.0;
                    for (int64_t k = blk * 32; k < blk * 32 + 32; ++k) {
                        double p = dec_elem(elem, arow, k) * dec_elem(elem, brow, k);
                        part += p;
                        pmag += fabs(p);
                    }
                    double sc = mxo_e8m0_value(sa[blk]) * mxo_e8m0_value(sb[blk]);
                    acc += part * sc;
                    mag += pmag * sc;
                }
            }
            if (exact) exact[i * N + n] = acc;
            if (bound) bound[i * N + n] = mag;
            if (out) out[i * N + n] = mxo_bf16_round(acc);
        }
    }
    return MXO_OK;
}

/* ------------------------------------------------------------------------- */
/* Gated activation + MXFP4 requant (NvMxf4f8Strategy fused_silu_quantize();
 * grouped_matmul_swiglu() is the same computation fused into the GEMM).
 * Input h: bf16 [nrows, 2I], column 2j = gate_j, column 2j+1 = up_j.
 *   y_j = bf16( g_j * u_j / (1 + exp(-g_j)) )   (fp64 then one rounding)
 * then MX E2M1 over j in blocks of 32: yq [nrows, I/2], ys [nrows, I/32].
 * y64 (optional, [nrows, I]) receives the unrounded fp64 y.                  */

static void silu_requant_row(const uint16_t* h, int64_t I, uint8_t* yq, uint8_t* ys, double* y64) {
    double blk[32];
    uint8_t codes[32];
    for (int64_t b = 0; b < I / 32; ++b) {
        for (int i = 0; i < 32; ++i) {
            int64_t j = b * 32 + i;
            double g = mxo_bf16_value(h[2 * j]);
            double u = mxo_bf16_value(h[2 * j + 1]);
            double y = g * u / (1.0 + exp(-g));
            if (y64) y64[j] = y;
            blk[i] = mxo_bf16_value(mxo_bf16_round(y));
        }
        ys[b] = quantize_block_mx(MXO_E2M1, blk, 32, codes);
        for (int i = 0; i < 16; ++i) yq[b * 16 + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
    }
}

/* Over the grouped rows of a [T, 2I] bf16 tensor (rows covered by a group). */
int mxo_silu_requant(const uint16_t* h, uint8_t* yq, uint8_t* ys, const uint32_t* off, int32_t G, int64_t T,
                     int64_t I, double* y64) {
    if (!h || !yq || !ys || !off || G < 0 || T < 0 || I <= 0 || (I % 32) != 0) return MXO_EINVAL;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        if (lo > hi) continue;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t t = lo; t < hi; ++t)
            silu_requant_row(h + t * 2 * I, I, yq + t * (I / 2), ys + t * (I / 32), y64 ? y64 + t * I : NULL);
    }
    return MXO_OK;
}

/* Fused gate/up GEMM + SwiGLU + requant on a list of rows: the MX GEMM of
 * mxo_gemm_rows against W [E, 2I, K] (rows interleaved gate, up), each output
 * rounded to bf16, then silu_requant_row.  gu_exact / gu_bound (optional,
 * [nrows, 2I]) receive the GEMM's unrounded values and magnitude sums. */
int mxo_gemm_swiglu_rows(int fmt, const uint8_t* a, const uint8_t* a_scale, const uint8_t* w,
                         const uint8_t* w_scale, const uint32_t* off, const int32_t* ids, int32_t G, int32_t E,
                         int64_t T, int64_t I, int64_t K, const int64_t* rows, int64_t nrows, uint8_t* yq,
                         uint8_t* ys, double* gu_exact, double* gu_bound, int32_t* group) {
    if (fmt != 1 && fmt != 2) return MXO_EINVAL;
    if (!yq || !ys || !rows || I <= 0 || (I % 32) != 0) return MXO_EINVAL;
    int64_t N = 2 * I;
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(nrows * N));
    int32_t* grp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrows > 0 ? nrows : 1));
    if (!h || !grp) {
        free(h);
        free(grp);
        return MXO_EINVAL;
    }
    int rc = mxo_gemm_rows(fmt, a, a_scale, w, w_scale, off, ids, G, E, T, N, K, rows, nrows, h, gu_exact,
                           gu_bound, grp);
    if (rc == MXO_OK) {
        for (int64_t i = 0; i < nrows; ++i) {
            if (group) group[i] = grp[i];
            if (grp[i] < 0) continue;
            silu_requant_row(h + i * N, I, yq + i * (I / 2), ys + i * (I / 32), NULL);
        }
    }
    free(grp);
    free(h);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* NVFP4 (NvMxf4f8Strategy: is_nvfp4, grouped_quantize(input_scale),
 * grouped_matmul(expert_scales); grouped_quantize_dynamic_scaled_fp4_async_
 * kernel, Args: sf_tensor, one tensor-level scale for each expert).  The pages
 * name the format and its scales but state no arithmetic; the readings taken
 * (listed with the design notes):
 *   - elements are E2M1 as in MXFP4, in blocks of 16 along K, each block with
 *     an E4M3 scale code;
 *   - sf, per expert, is the encode-side tensor scale: with amax the block's
 *     largest |x|, the block scale is s = e4m3(min(fl32(fl32(amax / 6) * sf),
 *     448)) and an element is e2m1(fl32(x * r)) with r = fl32(sf / s) (r = 0
 *     when s decodes to 0); so x ~ e2m1 * s / sf;
 *   - the grouped GEMM returns expert_scale[e] * sum_b sa[t,b] sb[e,n,b]
 *     sum_{k in b} qa[t,k] qb[e,n,k], expert_scale per expert (the epilogue
 *     factor, typically 1 / (sf_a * sf_b)).
 * Every fl32 step is one IEEE binary32 operation, round to nearest even.    */
static void quantize_row_nvfp4(const uint16_t* x, int64_t K, float sf, uint8_t* q, uint8_t* s) {
    for (int64_t b = 0; b < K / 16; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 16; ++i) {
            float a = fabsf((float)mxo_bf16_value(x[b * 16 + i]));
            if (a > amax) amax = a;
        }
        volatile float t = amax / 6.0f;
        volatile float u = t * sf;
        float uc = (u < 448.0f) ? u : 448.0f;
        uint8_t code = mxo_e4m3_encode((double)uc);
        s[b] = code;
        double sv = mxo_e4m3_value(code);
        volatile float r = 0.0f;
        if (sv != 0.0) r = sf / (float)sv;
        uint8_t c[16];
        for (int i = 0; i < 16; ++i) {
            volatile float v = (float)mxo_bf16_value(x[b * 16 + i]) * r;
            c[i] = mxo_e2m1_encode((double)v);
        }
        for (int i = 0; i < 8; ++i) q[b * 8 + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
    }
}

/* Rows of group g use sf[expert_ids[g]]; a group whose expert id lies outside
 * [0, E) or whose start exceeds its end is skipped; uncovered rows are left
 * as they were.  q u8 [T, K/2], scales u8 E4M3 [T, K/16].                    */
int mxo_quantize_nvfp4(const uint16_t* x, uint8_t* q, uint8_t* scales, const float* sf, const uint32_t* off,
                       const int32_t* ids, int32_t G, int32_t E, int64_t T, int64_t K) {
    if (!x || !q || !scales || !sf || !off || !ids || G < 0 || E <= 0 || T < 0 || K <= 0 || (K % 16) != 0)
        return MXO_EINVAL;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        if (lo > hi || ids[g] < 0 || ids[g] >= E) continue;
        const float f = sf[ids[g]];
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t t = lo; t < hi; ++t) quantize_row_nvfp4(x + t * K, K, f, q + t * (K / 2), scales + t * (K / 16));
    }
    return MXO_OK;
}

/* Grouped GEMM rows, NVFP4 operands (same outputs as mxo_gemm_rows).
 * a u8 [T, K/2], a_scale u8 E4M3 [T, K/16]; b u8 [E, N, K/2], b_scale u8
 * [E, N, K/16]; expert_scale fp32 [E].                                      */
int mxo_gemm_rows_nvfp4(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b, const uint8_t* b_scale,
                        const float* expert_scale, const uint32_t* off, const int32_t* ids, int32_t G, int32_t E,
                        int64_t T, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, uint16_t* out,
                        double* exact, double* bound, int32_t* group) {
    if (!a || !a_scale || !b || !b_scale || !expert_scale || !off || !ids || !rows) return MXO_EINVAL;
    if (G < 0 || E <= 0 || T < 0 || N <= 0 || K <= 0 || (K % 16) != 0) return MXO_EINVAL;
    const int64_t row_bytes = K / 2, nblk = K / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t t = rows[i];
        int32_t g = (t >= 0 && t < T) ? group_of_row(off, ids, G, E, T, t) : -1;
        if (group) group[i] = g;
        if (g < 0) continue;
        int32_t e = ids[g];
        const uint8_t* arow = a + t * row_bytes;
        const uint8_t* sa = a_scale + t * nblk;
        const double es = (double)expert_scale[e];
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* brow = b + ((int64_t)e * N + n) * row_bytes;
            const uint8_t* sb = b_scale + ((int64_t)e * N + n) * nblk;
            double acc = 0.0, mag = 0.0;
            for (int64_t blk = 0; blk < nblk; ++blk) {
                double part = 0.0, pmag = 0.0;
                for (int64_t k = blk * 16; k < blk * 16 + 16; ++k) {
                    double p = dec_elem(MXO_E2M1, arow, k) * dec_elem(MXO_E2M1, brow, k);
                    part += p;
                    pmag += fabs(p);
                }
                double sc = mxo_e4m3_value(sa[blk]) * mxo_e4m3_value(sb[blk]);
                acc += part * sc;
                mag += pmag * fabs(sc);
            }
            acc *= es;
            mag *= fabs(es);
            if (exact) exact[i * N + n] = acc;
            if (bound) bound[i * N + n] = mag;
            if (out) out[i * N + n] = mxo_bf16_round(acc);
        }
    }
    return MXO_OK;
}

/* NVFP4 gated activation + requant (NvMxf4f8Strategy, fused_silu_quantize();
 * grouped_matmul_swiglu(), Args input_scales and a_row_scales: one output-side
 * scale per expert, inverted by the strategy before the kernel sees it, and
 * an optional factor per routed row).  Readings: sf_y
 * below is that inverted (encode-side) scale; y_j = bf16(silu(g_j) u_j) as in
 * silu_requant_row, quantized to NVFP4 along j in blocks of 16 exactly as
 * quantize_row_nvfp4 does for a row of bf16 values.                        */
static void silu_requant_row_nvfp4(const uint16_t* h, int64_t I, float sf, uint8_t* yq, uint8_t* ys, double* y64) {
    uint16_t yb[16];
    for (int64_t b = 0; b < I / 16; ++b) {
        for (int i = 0; i < 16; ++i) {
            int64_t j = b * 16 + i;
            double g = mxo_bf16_value(h[2 * j]);
            double u = mxo_bf16_value(h[2 * j + 1]);
            double y = g * u / (1.0 + exp(-g));
            if (y64) y64[j] = y;
            yb[i] = mxo_bf16_round(y);
        }
        quantize_row_nvfp4(yb, 16, sf, yq + b * 8, ys + b);
    }
}

/* Rows of group g (expert id in [0, E)) use sf_y[ids[g]]; h bf16 [T, 2I];
 * yq [T, I/2], ys E4M3 [T, I/16]; uncovered rows are left as they were.   */
int mxo_silu_requant_nvfp4(const uint16_t* h, uint8_t* yq, uint8_t* ys, const float* sf_y, const uint32_t* off,
                           const int32_t* ids, int32_t G, int32_t E, int64_t T, int64_t I, double* y64) {
    if (!h || !yq || !ys || !sf_y || !off || !ids || G < 0 || E <= 0 || T < 0 || I <= 0 || (I % 16) != 0)
        return MXO_EINVAL;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        if (lo > hi || ids[g] < 0 || ids[g] >= E) continue;
        const float f = sf_y[ids[g]];
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t t = lo; t < hi; ++t)
            silu_requant_row_nvfp4(h + t * 2 * I, I, f, yq + t * (I / 2), ys + t * (I / 16), y64 ? y64 + t * I : NULL);
    }
    return MXO_OK;
}

/* Fused NVFP4 gate/up GEMM + SwiGLU + NVFP4 requant on a list of rows: the
 * NVFP4 GEMM (expert scale included), times the optional bf16 row scale
 * rs[t] (reading: it multiplies in with the expert scale, ahead of the
 * activation; grouped_matmul_swiglu(), Args a_row_scales), each
 * output rounded to bf16, then silu_requant_row_nvfp4 with sf_y[e].
 * gu_exact / gu_bound include the row scale.                                */
int mxo_gemm_swiglu_rows_nvfp4(const uint8_t* a, const uint8_t* a_scale, const uint8_t* w, const uint8_t* w_scale,
                               const float* expert_scale, const uint16_t* row_scale, const float* sf_y,
                               const uint32_t* off, const int32_t* ids, int32_t G, int32_t E, int64_t T, int64_t I,
                               int64_t K, const int64_t* rows, int64_t nrows, uint8_t* yq, uint8_t* ys,
                               double* gu_exact, double* gu_bound, int32_t* group) {
    if (!yq || !ys || !rows || !sf_y || I <= 0 || (I % 16) != 0) return MXO_EINVAL;
    int64_t N = 2 * I;
    double* ex = (double*)malloc(sizeof(double) * (size_t)(nrows * N > 0 ? nrows * N : 1));
    double* bd = (double*)malloc(sizeof(double) * (size_t)(nrows * N > 0 ? nrows * N : 1));
    int32_t* grp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrows > 0 ? nrows : 1));
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N > 0 ? N : 1));
    if (!ex || !bd || !grp || !h) {
        free(ex);
        free(bd);
        free(grp);
        free(h);
        return MXO_EINVAL;
    }
    int rc = mxo_gemm_rows_nvfp4(a, a_scale, w, w_scale, expert_scale, off, ids, G, E, T, N, K, rows, nrows, NULL,
                                 ex, bd, grp);
    if (rc == MXO_OK) {
        for (int64_t i = 0; i < nrows; ++i) {
            if (group) group[i] = grp[i];
            if (grp[i] < 0) continue;
            const double rs = row_scale ? mxo_bf16_value(row_scale[rows[i]]) : 1.0;
            for (int64_t n = 0; n < N; ++n) {
                const double v = ex[i * N + n] * rs;
                h[n] = mxo_bf16_round(v);
                if (gu_exact) gu_exact[i * N + n] = v;
                if (gu_bound) gu_bound[i * N + n] = bd[i * N + n] * fabs(rs);
            }
            silu_requant_row_nvfp4(h, I, sf_y[ids[grp[i]]], yq + i * (I / 2), ys + i * (I / 16), NULL);
        }
    }
    free(h);
    free(grp);
    free(bd);
    free(ex);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Padded / slot-strided MX scale layouts (grouped_quantize_dynamic_scaled_fp4_
 * async_kernel: scales_offsets, the per-expert offsets into the scale tensor,
 * found with row_offsets by binary search; NvMxf4f8Strategy grouped_quantize(),
 * its padded scale layout and scales_offset; Struct_ep_dispatch_mxfp4: the
 * fixed-stride slot layout [n_local_experts * max_padded_M, K_SCALES]).
 * Reading: routed row t of group g keeps its K/32 scale bytes in row
 * soff[g] + (t - row_offsets[g]) of a scale tensor of S rows (the slot layout
 * is soff[g] = expert_ids[g] * max_padded_M); a row whose scale row lies at or
 * past S is left untouched (codes included); scale rows nothing maps to are
 * never written.  MX formats only (fmt 1, 2).                               */
int mxo_quantize_padded(int fmt, const uint16_t* x, uint8_t* q, uint8_t* scales, const uint32_t* soff, int64_t S,
                        const uint32_t* off, int32_t G, int64_t T, int64_t K) {
    if (!x || !q || !scales || !soff || !off || G < 0 || T < 0 || S < 0 || K <= 0 || (K % 32) != 0) return MXO_EINVAL;
    if (fmt != 1 && fmt != 2) return MXO_EINVAL;
    const int elem = fmt == 2 ? MXO_E2M1 : MXO_E4M3;
    const int64_t row_bytes = fmt == 2 ? K / 2 : K;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        if (lo > hi) continue;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t t = lo; t < hi; ++t) {
            const int64_t srow = (int64_t)soff[g] + (t - lo);
            if (srow >= S) continue;
            quantize_row_mx(elem, x + t * K, K, q + t * row_bytes, scales + srow * (K / 32));
        }
    }
    return MXO_OK;
}

/* NVFP4 in the same padded / slot-strided layout (the scales_offsets argument
 * of grouped_quantize_dynamic_scaled_fp4_async_kernel covers NVFP4 as well):
 * routed row t of taken group g (expert id in [0, E)) is quantized as in
 * mxo_quantize_nvfp4 with tensor scale sf[ids[g]], its K/16 E4M3 scale bytes
 * going to row soff[g] + (t - row_offsets[g]) of a [S, K/16] tensor; a row
 * whose scale row lies at or past S is left untouched (codes included).    */
int mxo_quantize_nvfp4_padded(const uint16_t* x, uint8_t* q, uint8_t* scales, const float* sf,
                              const uint32_t* soff, int64_t S, const uint32_t* off, const int32_t* ids, int32_t G,
                              int32_t E, int64_t T, int64_t K) {
    if (!x || !q || !scales || !sf || !soff || !off || !ids || G < 0 || E <= 0 || T < 0 || S < 0 || K <= 0 ||
        (K % 16) != 0)
        return MXO_EINVAL;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        if (lo > hi || ids[g] < 0 || ids[g] >= E) continue;
        const float f = sf[ids[g]];
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t t = lo; t < hi; ++t) {
            const int64_t srow = (int64_t)soff[g] + (t - lo);
            if (srow >= S) continue;
            quantize_row_nvfp4(x + t * K, K, f, q + t * (K / 2), scales + srow * (K / 16));
        }
    }
    return MXO_OK;
}

/* Grouped GEMM rows with A's scales in such a layout: the dense A scales are
 * gathered row by row through the map above, then mxo_gemm_rows runs; a row
 * whose scale row lies at or past Sa is reported uncovered (group -1).     */
int mxo_gemm_rows_padded(int fmt, const uint8_t* a, const uint8_t* a_scale, const uint32_t* asoff, int64_t Sa,
                         const uint8_t* b, const uint8_t* b_scale, const uint32_t* off, const int32_t* ids, int32_t G,
                         int32_t E, int64_t T, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, uint16_t* out,
                         double* exact, double* bound, int32_t* group) {
    if (!a_scale || !asoff || Sa < 0 || (fmt != 1 && fmt != 2) || K <= 0 || (K % 32) != 0 || T < 0 || G < 0)
        return MXO_EINVAL;
    const int64_t nblk = K / 32;
    uint8_t* dense = (uint8_t*)calloc((size_t)(T > 0 ? T : 1) * (size_t)nblk, 1);
    int32_t* grp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrows > 0 ? nrows : 1));
    if (!dense || !grp) {
        free(dense);
        free(grp);
        return MXO_EINVAL;
    }
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t t = rows[i];
        const int32_t g = (t >= 0 && t < T) ? group_of_row(off, ids, G, E, T, t) : -1;
        grp[i] = g;
        if (g < 0) continue;
        int64_t lo, hi;
        group_range(off, g, T, &lo, &hi);
        const int64_t srow = (int64_t)asoff[g] + (t - lo);
        if (srow >= Sa) {
            grp[i] = -1;
            continue;
        }
        memcpy(dense + t * nblk, a_scale + srow * nblk, (size_t)nblk);
    }
    int rc = mxo_gemm_rows(fmt, a, dense, b, b_scale, off, ids, G, E, T, N, K, rows, nrows, out, exact, bound, group);
    if (rc == MXO_OK && group)
        for (int64_t i = 0; i < nrows; ++i)
            if (grp[i] < 0) group[i] = -1;
    free(grp);
    free(dense);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Array forms of the scalar codecs, for exhaustive checks.                    */
void mxo_e4m3_encode_array(const double* v, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = mxo_e4m3_encode(v[i]);
}
void mxo_e2m1_encode_array(const double* v, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = mxo_e2m1_encode(v[i]);
}
/* MoE combine after the down-projection (grouped_matmul_rowwise_dynamic_
 * scaled_fp8, Parameters: elementwise_lambda_fn -- the output epilogue at
 * (global_row, n); NvMxf4f8Strategy, the EP-combine path; the pages do not
 * define the combine, and the reading taken is the router-weighted sum):
 *   exact[t, n] = sum_k w[t*top_k + k] * y[row_of_slot[t*top_k + k], n]
 * over the slots whose row lies in [0, T) -- each product of an fp32 weight
 * and a bf16 value is exact in fp64 --, bound[t, n] = the same sum of
 * |products|, out = bf16 round-to-nearest-even of exact.  Any of out /
 * exact / bound may be NULL.                                               */
int mxo_combine(const uint16_t* y, int64_t T, int64_t H, const int32_t* row_of_slot, const float* w,
                int64_t ntok, int32_t top_k, uint16_t* out, double* exact, double* bound) {
    if (H <= 0 || T < 0 || ntok < 0 || top_k < 1 || !row_of_slot || !w) return MXO_EINVAL;
    if (T > 0 && !y) return MXO_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t) {
        for (int64_t n = 0; n < H; ++n) {
            double e = 0.0, b = 0.0;
            for (int32_t k = 0; k < top_k; ++k) {
                const int32_t r = row_of_slot[t * top_k + k];
                if (r < 0 || (int64_t)r >= T) continue;
                const double p = (double)w[t * top_k + k] * mxo_bf16_value(y[(int64_t)r * H + n]);
                e += p;
                b += fabs(p);
            }
            if (out) out[t * H + n] = mxo_bf16_round(e);
            if (exact) exact[t * H + n] = e;
            if (bound) bound[t * H + n] = b;
        }
    }
    return MXO_OK;
}

void mxo_bf16_round_array(const double* v, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = mxo_bf16_round(v[i]);
}
void mxo_e4m3_value_array(const uint8_t* c, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = mxo_e4m3_value(c[i]);
}
void mxo_e2m1_value_array(const uint8_t* c, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = mxo_e2m1_value(c[i]);
}
