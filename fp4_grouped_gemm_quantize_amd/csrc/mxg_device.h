// mxg_device.h -- gfx950 device helpers shared by the quantize and GEMM kernels:
// bit-level element encoders, bf16 rounding, wave reductions and the group
// bookkeeping every kernel does on row_offsets / expert_ids.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

constexpr int kWave = 64;
constexpr int kMaxGroups = 1024;

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the upper half of binary32; fp32 -> bf16 rounds to
// nearest, ties to even (overflow goes to infinity as IEEE rounding does, a
// NaN keeps its upper half with the quiet bit set).  The conversion is the
// hardware packed convert (v_cvt_pk_bf16_f32), checked on gfx950 against the
// integer form of that rounding -- u += 0x7fff + ((u >> 16) & 1), keep the
// upper half; NaN: (u >> 16) | 0x40 -- for all 2^32 fp32 inputs, bit for bit.
// One instruction instead of five; the GEMM epilogues and the SwiGLU requant
// round every output through it.
typedef float mxg_f2v __attribute__((ext_vector_type(2)));
typedef __bf16 mxg_b2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    const mxg_b2v b = __builtin_convertvector((mxg_f2v){lo, hi}, mxg_b2v);
    uint32_t r;
    __builtin_memcpy(&r, &b, 4);
    return r;
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    const __bf16 b = (__bf16)f;
    uint16_t r;
    __builtin_memcpy(&r, &b, 2);
    return r;
}

// ---------------------------------------------------------------------------
// OCP OFP8 E4M3 ("fn": no infinities, max 448) from fp32, round to nearest
// even, saturating.  Bit manipulation on the binary32 pattern:
//   |v| >= 448           -> 0x7e
//   |v| <  2^-6          -> subnormal: m = rne(|v| * 2^9) in 0..8 (8 is 0x08)
//   otherwise            -> round the pattern at bit 20 (3 mantissa bits kept,
//                           carries run into the exponent), rebias 127 -> 7.
__device__ __forceinline__ uint32_t enc_e4m3(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t s = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    // (the min() keeps the unused branch's float->int conversion in range)
    uint32_t sub = (uint32_t)__builtin_rintf(fminf(__uint_as_float(a), 0.015625f) * 512.0f);
    uint32_t nrm = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    uint32_t c = a < 0x3c800000u ? sub : nrm;
    c = a >= 0x43e00000u ? 0x7eu : c;
    return s | c;
}

// OCP MX E2M1 (max 6) from fp32, round to nearest even, saturating.
//   |v| >= 6  -> 7;  |v| < 1 -> rne(2|v|) in 0..2;  else round at bit 22.
__device__ __forceinline__ uint32_t enc_e2m1(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t s = (u >> 28) & 0x8u;
    uint32_t a = u & 0x7fffffffu;
    uint32_t sub = (uint32_t)__builtin_rintf(fminf(__uint_as_float(a), 1.0f) * 2.0f);
    uint32_t nrm = ((a + 0x1fffffu + ((a >> 22) & 1u)) >> 22) - (126u << 1);
    uint32_t c = a < 0x3f800000u ? sub : nrm;
    c = a >= 0x40c00000u ? 7u : c;
    return s | c;
}

// floor(log2(a)) of a positive finite fp32 (normal or subnormal), exactly.
__device__ __forceinline__ int floor_log2_f32(float a) {
    uint32_t u = __float_as_uint(a);
    int e = (int)(u >> 23);
    if (e != 0) return e - 127;
    uint32_t m = u & 0x7fffffu;
    return (31 - __clz(m)) - 149;
}

// MX shared exponent of a block with maximum magnitude amax (OCP MX v1.0):
// X = clamp(floor(log2 amax) - emax_elem, -127, 127); the E8M0 code is X+127,
// and an all-zero block gets code 0 (elements are then signed zeros anyway).
__device__ __forceinline__ int mx_shared_exp(float amax, int emax_elem) {
    if (amax == 0.0f) return -127;
    int x = floor_log2_f32(amax) - emax_elem;
    return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// ---------------------------------------------------------------------------
// Wave reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Gated activation in fp32, the one formula both the fused GEMM epilogue and
// the standalone activation kernel use: silu(g) * u with silu(z) = z/(1+e^-z).
__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// ---------------------------------------------------------------------------
// Group bookkeeping.  Group g is taken when its (clamped) start does not
// exceed its end and, if experts are checked (num_experts > 0), its id is in
// range; its rows are [lo, hi).
struct GroupRange {
    int64_t lo, hi;
};

__device__ __forceinline__ GroupRange group_range(const uint32_t* off, const int32_t* ids, int g, int64_t T,
                                                  int num_experts) {
    int64_t lo = (int64_t)off[g], hi = (int64_t)off[g + 1];
    lo = lo < T ? lo : T;
    hi = hi < T ? hi : T;
    if (hi < lo) hi = lo;
    if (num_experts > 0) {
        int e = ids[g];
        if (e < 0 || e >= num_experts) hi = lo;
    }
    return {lo, hi};
}

// Whether any taken group covers row t.  The whole wave cooperates: lane i
// tests groups i, i+64, ...; the result is wave-uniform.  Offsets are read
// from LDS (s_off holds row_offsets[0..G]).
__device__ __forceinline__ bool wave_row_covered(const uint32_t* s_off, int G, int64_t T, int64_t t) {
    int lane = threadIdx.x & (kWave - 1);
    bool hit = false;
    for (int g = lane; g < G; g += kWave) {
        int64_t lo = (int64_t)s_off[g], hi = (int64_t)s_off[g + 1];
        lo = lo < T ? lo : T;
        hi = hi < T ? hi : T;
        hit |= (t >= lo) && (t < hi);
    }
    return __any(hit);
}

// 16 bytes of a stream that is read once, loaded with the nontemporal hint.
// Measured on MI355X: the grouped quantize of 537 MB of BF16 rows runs ~17 %
// faster than with ordinary loads (FP8 rowwise 155 -> 129 us, MXFP4 133 ->
// 115 us, same bytes out).  Nontemporal stores of the codes gave nothing on
// top; the gathered quantize (token rows shared by several slots), the
// SwiGLU requant and the combine were as fast or faster with ordinary loads
// and keep them.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    typedef unsigned u4v __attribute__((ext_vector_type(4)));
    const u4v t = __builtin_nontemporal_load(static_cast<const u4v*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// 16 bytes written with the nontemporal hint (an output nothing in the same
// kernel reads back).  The GEMM's BF16 output pieces use it: ~1 % faster on
// the ragged FP8 and MXFP8 GEMMs, same bytes.
__device__ __forceinline__ void store_stream16(void* p, const uint4& v) {
    typedef unsigned u4v __attribute__((ext_vector_type(4)));
    u4v t;
    t.x = v.x;
    t.y = v.y;
    t.z = v.z;
    t.w = v.w;
    __builtin_nontemporal_store(t, static_cast<u4v*>(p));
}

// Unpack a 16-byte vector of 8 bf16 into fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
        f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
}

// ---------------------------------------------------------------------------
// Hardware packing converts.  Checked exhaustively on gfx950 against the
// bit-level encoders above: v_cvt_pk_fp8_f32 equals enc_e4m3 for every fp32
// input of magnitude <= 448 + 1/2 ulp (beyond that it does not saturate, so
// callers clamp first), and v_cvt_scalef32_pk_fp4_f32 with scale 1 equals
// enc_e2m1 for every fp32 input, saturation included.  The first element of
// each pair lands in the low byte / low nibble.
__device__ __forceinline__ uint2 pack8_e4m3(const float* f) {
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0u, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0u, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
    return make_uint2(lo, hi);
}

__device__ __forceinline__ uint32_t pack8_e2m1(const float* f) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[0], f[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], 1.0f, 3);
    return w;
}

// ---------------------------------------------------------------------------
// MX: 4 lanes x 8 elements form one 32-element block.  Given the 8 values of
// this lane, returns the block's shared exponent X (after the 4-lane
// reduction) and the lane's packed codes of x * 2^-X (e4m3: 8 bytes; e2m1:
// 8 nibbles in word .x).  Every lane of the 4-lane group must call it.
template <bool FP4>
__device__ __forceinline__ int mx_encode8(const float* f, uint2& packed) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    const int X = mx_shared_exp(amax, FP4 ? 2 : 8);
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        e[i] = ldexpf(f[i], -X);  // exact power-of-two shift
        if (!FP4) e[i] = fminf(fmaxf(e[i], -448.0f), 448.0f);  // saturate (the convert does not)
    }
    if (FP4) packed = make_uint2(pack8_e2m1(e), 0u);
    else packed = pack8_e4m3(e);
    return X;
}

// Store one lane's 8 codes (unit `idx` of 8 elements in the row) and, from the
// first lane of the block, the block's E8M0 scale.
template <bool FP4>
__device__ __forceinline__ void mx_store8(const uint2& packed, int X, uint8_t* qrow, uint8_t* srow, int64_t idx,
                                          int lane) {
    if (FP4) *reinterpret_cast<uint32_t*>(qrow + idx * 4) = packed.x;
    else *reinterpret_cast<uint2*>(qrow + idx * 8) = packed;
    if ((lane & 3) == 0) srow[idx >> 2] = (uint8_t)(X + 127);
}

// ---------------------------------------------------------------------------
// NVFP4: 2 lanes x 8 elements form one 16-element block.  With sf the
// group's encode-side tensor scale: block scale code = e4m3(min(fl32(
// fl32(amax / 6) * sf), 448)), element code = e2m1(fl32(x * r)), r =
// fl32(sf / s) with s the scale code's value (r = 0 when s is 0).  Each step
// is one IEEE binary32 operation; the e4m3 code comes from the convert above
// (exact up to 448) and its value from the exact fp8 -> fp32 convert.
// Returns the lane's 8 packed codes; every lane of the pair must call it.
__device__ __forceinline__ uint32_t nv_encode8(const float* f, float sf, uint32_t& scode) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    const float t = amax / 6.0f;
    const float u = t * sf;
    const float uc = u < 448.0f ? u : 448.0f;
    scode = __builtin_amdgcn_cvt_pk_fp8_f32(uc, 0.0f, 0u, false) & 0xffu;
    const float s = __builtin_amdgcn_cvt_f32_fp8((int)scode, 0);
    const float r = s == 0.0f ? 0.0f : sf / s;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = f[i] * r;
    return pack8_e2m1(v);
}

// The group covering row t whose expert id lies in [0, E) (the lowest such
// group; with ids == nullptr any covering group), or -1.  Wave-cooperative,
// result wave-uniform; offsets from LDS.
__device__ __forceinline__ int wave_row_group(const uint32_t* s_off, const int32_t* ids, int G, int E, int64_t T,
                                              int64_t t) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int g0 = 0; g0 < G; g0 += kWave) {
        const int g = g0 + lane;
        bool hit = false;
        if (g < G) {
            int64_t lo = (int64_t)s_off[g], hi = (int64_t)s_off[g + 1];
            lo = lo < T ? lo : T;
            hi = hi < T ? hi : T;
            if (t >= lo && t < hi) {
                if (ids) {
                    const int e = ids[g];
                    hit = e >= 0 && e < E;
                } else {
                    hit = true;
                }
            }
        }
        const uint64_t m = __ballot(hit);
        if (m) return g0 + __builtin_ctzll(m);
    }
    return -1;
}

}  // namespace mxg
