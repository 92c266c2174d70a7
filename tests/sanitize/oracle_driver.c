/* Runs every oracle routine on small inputs with the edge cases of the
 * routing contract (empty, inverted and out-of-range groups, offsets past the
 * rows, dropped slots, rows outside the tensor) and of the encodings (zeros,
 * subnormals, saturating values, infinities and NaNs), for an
 * AddressSanitizer / UndefinedBehaviorSanitizer build.  The oracle source is
 * compiled into this program.  Prints a checksum; exits 0 when every call
 * returned its expected status. */
#include "../../oracle/oracle.c"

#include <stdio.h>

static uint32_t lcg_state = 12345u;
static uint32_t lcg(void) {
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return lcg_state >> 8;
}

#define T 37
#define K 96
#define KB (K / 32)
#define E 3
#define N 64
#define I 32

static int fails = 0;
#define EXPECT(cond)                                                 \
    do {                                                             \
        if (!(cond)) {                                               \
            fprintf(stderr, "expectation failed line %d\n", __LINE__); \
            ++fails;                                                 \
        }                                                            \
    } while (0)

int main(void) {
    static uint16_t x[T * K], h[T * 2 * I];
    static uint8_t q[T * K], s8[T * KB], b[E * N * K], bs[E * N * KB], w[E * 2 * I * K], ws[E * 2 * I * KB];
    static float s32[T], bs32[E * N];
    static uint8_t yq[T * I], ys[T * I];
    static uint16_t out[(T + 2) * N];
    static double ex[(T + 2) * N], bd[(T + 2) * N], y64[T * I];
    static int32_t grp[T + 2];
    double sum = 0.0;
    for (int i = 0; i < T * K; ++i) {
        uint32_t r = lcg();
        uint16_t v = (uint16_t)r;
        if (i % 97 == 0) v = 0x7F80 | (uint16_t)(r & 0x8000);        /* infinities */
        if (i % 101 == 0) v = 0x7FC1;                                 /* a NaN */
        if (i % 7 == 0) v &= 0x807F;                                  /* zeros and subnormals */
        x[i] = v;
    }
    for (int i = 0; i < T * 2 * I; ++i) h[i] = (uint16_t)(lcg() & 0xBFFF);
    /* groups: normal, empty, inverted, bad expert id, past the rows */
    const uint32_t off[6] = {0, 9, 9, 5, 30, 41};
    const int32_t ids[5] = {0, 1, 2, 7, 1};
    const int32_t G = 5;
    for (int fmt = 0; fmt <= 2; ++fmt) {
        EXPECT(mxo_quantize(fmt, x, q, fmt == 0 ? (void*)s32 : (void*)s8, off, G, T, K) == MXO_OK);
        for (int i = 0; i < T; ++i) sum += q[i * (fmt == 2 ? K / 2 : K)];
    }
    EXPECT(mxo_quantize(3, x, q, s8, off, G, T, K) != MXO_OK);
    EXPECT(mxo_quantize(1, x, q, s8, off, G, T, 40) != MXO_OK);
    /* gather: indices past the sources and negative ones are skipped */
    int32_t idx[T];
    for (int i = 0; i < T; ++i) idx[i] = (i % 11 == 0) ? -1 : (int32_t)(lcg() % (2 * T));
    for (int fmt = 0; fmt <= 2; ++fmt)
        EXPECT(mxo_quantize_gather(fmt, x, T / 2, idx, 2, q, fmt == 0 ? (void*)s32 : (void*)s8, off, G, T, K) ==
               MXO_OK);
    /* GEMM rows, including rows outside the tensor */
    for (int i = 0; i < E * N * K; ++i) b[i] = (uint8_t)(lcg() & 0xF7);
    for (int i = 0; i < E * N * KB; ++i) bs[i] = (uint8_t)(110 + lcg() % 30);
    for (int i = 0; i < E * N; ++i) bs32[i] = (float)(lcg() % 1000) / 997.0f;
    int64_t rows[T + 2];
    for (int i = 0; i < T; ++i) rows[i] = i;
    rows[T] = -1;
    rows[T + 1] = T;
    for (int fmt = 0; fmt <= 2; ++fmt) {
        mxo_quantize(fmt, x, q, fmt == 0 ? (void*)s32 : (void*)s8, off, G, T, K);
        EXPECT(mxo_gemm_rows(fmt, q, fmt == 0 ? (void*)s32 : (void*)s8, b, fmt == 0 ? (void*)bs32 : (void*)bs, off,
                             ids, G, E, T, N, K, rows, T + 2, out, ex, bd, grp) == MXO_OK);
        EXPECT(grp[T] == -1 && grp[T + 1] == -1);
        for (int i = 0; i < T * N; ++i) sum += out[i] * 1e-9;
    }
    /* gated activation + MXFP4 requant, chained and fused */
    EXPECT(mxo_silu_requant(h, yq, ys, off, G, T, I, y64) == MXO_OK);
    for (int i = 0; i < E * 2 * I * K; ++i) w[i] = (uint8_t)lcg();
    for (int i = 0; i < E * 2 * I * KB; ++i) ws[i] = (uint8_t)(115 + lcg() % 20);
    mxo_quantize(2, x, q, s8, off, G, T, K);
    EXPECT(mxo_gemm_swiglu_rows(2, q, s8, w, ws, off, ids, G, E, T, I, K, rows, T, yq, ys, ex, bd, grp) == MXO_OK);
    /* NVFP4 */
    static uint8_t s16[T * (K / 16)], bs16[E * N * (K / 16)], ws16[E * 2 * I * (K / 16)];
    const float sf[E] = {100.0f, 300.0f, 2688.0f}, es[E] = {0.5f, 1.0f, 1e-3f}, sfy[E] = {400.0f, 1.0f, 20.0f};
    static uint16_t rs[T];
    for (int i = 0; i < T; ++i) rs[i] = (uint16_t)(0x3F80 + (lcg() & 0x3F));
    for (int i = 0; i < E * N * (K / 16); ++i) bs16[i] = (uint8_t)(lcg() % 0x7E);
    for (int i = 0; i < E * 2 * I * (K / 16); ++i) ws16[i] = (uint8_t)(lcg() % 0x7E);
    EXPECT(mxo_quantize_nvfp4(x, q, s16, sf, off, ids, G, E, T, K) == MXO_OK);
    EXPECT(mxo_gemm_rows_nvfp4(q, s16, b, bs16, es, off, ids, G, E, T, N, K, rows, T + 2, out, ex, bd, grp) ==
           MXO_OK);
    EXPECT(mxo_silu_requant_nvfp4(h, yq, ys, sfy, off, ids, G, E, T, I, y64) == MXO_OK);
    EXPECT(mxo_gemm_swiglu_rows_nvfp4(q, s16, w, ws16, es, rs, sfy, off, ids, G, E, T, I, K, rows, T, yq, ys, ex, bd,
                                      grp) == MXO_OK);
    /* padded scales: one slot cut short by the end of the scale tensor */
    const uint32_t soff[5] = {0, 16, 32, 48, 20};
    static uint8_t sp[64 * KB];
    EXPECT(mxo_quantize_padded(1, x, q, sp, soff, 40, off, G, T, K) == MXO_OK);
    EXPECT(mxo_gemm_rows_padded(2, q, sp, soff, 40, b, bs, off, ids, G, E, T, N, K, rows, T + 2, out, ex, bd, grp) ==
           MXO_OK);
    /* combine with dropped slots */
    int32_t ros[2 * T];
    float wt[2 * T];
    for (int i = 0; i < 2 * T; ++i) {
        ros[i] = (int32_t)(lcg() % (T + 4)) - 2;
        wt[i] = (float)(lcg() % 1000) / 333.0f;
    }
    EXPECT(mxo_combine(h, T, 2 * I, ros, wt, T, 2, out, ex, bd) == MXO_OK);
    /* scalar codecs over every code and a sweep of doubles */
    for (int c = 0; c < 256; ++c) {
        const double v = mxo_e4m3_value((uint8_t)c), s = mxo_e8m0_value((uint8_t)c);
        if (!isnan(v)) sum += v;
        if (!isnan(s)) sum += s * 1e-40;
    }
    for (int c = 0; c < 16; ++c) sum += mxo_e2m1_value((uint8_t)c);
    for (int i = -1200; i <= 1200; ++i) {
        const double v = ldexp(1.0 + (i & 7) / 8.0, i / 8);
        sum += mxo_e4m3_encode(v) + mxo_e2m1_encode(-v) + mxo_bf16_round(v) * 1e-6;
    }
    sum += (double)(mxo_bf16_round(INFINITY) + mxo_bf16_round(NAN) + mxo_e4m3_encode(NAN) + mxo_e2m1_encode(INFINITY));
    printf("checksum %.6f fails %d\n", sum, fails);
    return fails == 0 ? 0 : 1;
}
