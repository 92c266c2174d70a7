// quantize.hip -- grouped dynamic quantization of BF16 rows (FP8 rowwise, MXFP8,
// MXFP4) and the standalone SwiGLU + MXFP4 requant, for gfx950.
//
// Both passes are HBM-bound streams.  One wave owns one row at a time: each
// lane loads 16-byte vectors (8 bf16), so a wave reads 1 KiB per instruction,
// fully coalesced.  Waves are persistent (the grid is sized to the resident
// capacity) and load the next row they own while they encode the current one,
// so row loads stay in flight behind the arithmetic.  MX block maxima are
// reduced across the 4 lanes that share a 32-element block; the rowwise
// maximum across the whole wave.  Codes are packed by the hardware converts
// and written as 8-byte (e4m3) or 4-byte (e2m1) stores per lane.
//
// (grouped_quantize_dynamic_scaled_fp4_async_kernel, description;
//  NvMxf4f8Strategy, grouped_quantize() / fused_silu_quantize().)
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;  // one row per wave at a time
constexpr int kVecElems = 8;                      // bf16 per 16-byte vector
constexpr int kChunk = kWave * kVecElems;         // 512 elements per wave-wide load

__device__ __forceinline__ void load_offsets(uint32_t* s_off, const uint32_t* off, int G) {
    for (int i = threadIdx.x; i <= G; i += blockDim.x) s_off[i] = off[i];
    __syncthreads();
}

// The rowwise quotient x / scale (scale > 0) as IEEE binary32 division rounds
// it, computed as one fp64 product with the fp64 reciprocal of the scale
// followed by the binary64 -> binary32 rounding.  Equality with the binary32
// division was checked exhaustively on gfx950 for every bf16 amax (scale =
// amax / 448) and every bf16 x with |x| <= amax.
__device__ __forceinline__ float div_by_scale(float x, double inv_scale) { return (float)((double)x * inv_scale); }

// Gathered input (grouped_quantize(): indices, indices_divisor): routed row
// t reads source row indices[t] / divisor of x, which has nsrc rows; a row
// whose index is negative or names no source row is skipped (left
// untouched), so no read leaves x.  Without GATHER, row t reads row t.
struct Gather {
    const int32_t* idx;
    int32_t div;
    int64_t nsrc;
};

// NVFP4 (format 3): the rows of group g use tensor scale sf[ids[g]]; a group
// whose expert id lies outside [0, E) is skipped.
struct NvScales {
    const int32_t* ids;
    const float* sf;
    int E;
};

// Padded MX scale layout (grouped_quantize_dynamic_scaled_fp4_async_kernel:
// scales_offsets): the scales of group g's row t go to row soff[g] + (t -
// row_offsets[g]) of a scale tensor of S rows; a row mapped at or past S is
// skipped.  soff == nullptr: the dense layout (scale row t).
struct Pad {
    const uint32_t* soff;
    int64_t S;
};

// Token-major input (the gathered quantize read through the inverse slot map
// that the combine takes): unit rows are the ntok token rows of x; token s is
// encoded once and its codes and scales go to every routed row
// ros[s * top_k + k] that lies in [0, T) and is covered by a group (a routed
// row is a copy of its token's row).  top_k <= 64: lane k holds slot k.
struct Scatter {
    const int32_t* ros;
    int top_k;
    int64_t ntok;
};

// Scale row of row t under the layout, or -1 when the row is not written.
__device__ __forceinline__ int64_t scale_row(const Pad& pd, const uint32_t* s_off, int G, int64_t T, int64_t t) {
    if (!pd.soff) return wave_row_covered(s_off, G, T, t) ? t : -1;
    const int g = wave_row_group(s_off, nullptr, G, 0, T, t);
    if (g < 0) return -1;
    const int64_t lo = (int64_t)s_off[g] < T ? (int64_t)s_off[g] : T;
    const int64_t r = (int64_t)pd.soff[g] + (t - lo);
    return r < pd.S ? r : -1;
}

template <bool GATHER>
__device__ __forceinline__ int64_t source_row(const Gather& g, int64_t t) {
    if constexpr (!GATHER) {
        return t;
    } else {
        const int32_t v = g.idx[t];
        if (v < 0) return -1;
        const int64_t s = v / g.div;
        return s < g.nsrc ? s : -1;
    }
}

// ---------------------------------------------------------------------------
// Work units held in registers: a wave owns one unit at a time.  FP8 rowwise:
// a unit is a whole row (K <= NC * 512), since its scale needs the row's
// maximum.  MX and NVFP4 blocks are independent along K, so a row is split
// into nseg segments of NC * 512 elements (the last one may be shorter) and
// each segment is a unit: long rows then need no more than 8 chunks of
// registers per buffer, which keeps 4 waves per SIMD resident (measured: K =
// 7168 as one 14-chunk unit reached 63 % of HBM bandwidth, at 2 waves per
// SIMD).
// FMT: 0 = FP8 rowwise (scale = amax / 448, code = e4m3(x / scale)),
//      1 = MXFP8, 2 = MXFP4, 3 = NVFP4.
template <int FMT, int NC, bool GATHER, bool SCATTER>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const uint16_t* __restrict__ x,
                                                                 uint8_t* __restrict__ q, void* __restrict__ scales,
                                                                 const uint32_t* __restrict__ off, int G,
                                                                 int64_t T, int64_t K, int nseg, Gather ga,
                                                                 NvScales nv, Pad pd, Scatter sc) {
    static_assert(!(GATHER && SCATTER) && (!SCATTER || FMT <= 2), "scatter: FP8 rowwise / MX, no gather");
    __shared__ uint32_t s_off[kMaxGroups + 1];
    load_offsets(s_off, off, G);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    constexpr int64_t kSegElems = (int64_t)NC * kChunk;
    const int64_t units = (SCATTER ? sc.ntok : T) * nseg;  // unit rows: tokens when scattering

    // Unit u: row t = u / nseg, elements [e0, e0 + 8 * nvec).
    struct Unit {
        int64_t t, e0, sr;  // sr: source row of x (-1: none)
        int nvec;           // 16-byte vectors in the unit
    };
    auto unit = [&](int64_t u) {
        Unit w{0, 0, -1, 0};
        if (u >= units) return w;
        w.t = nseg == 1 ? u : u / nseg;
        w.e0 = (u - w.t * nseg) * kSegElems;
        const int64_t left = K - w.e0;
        w.nvec = (int)((left < kSegElems ? left : kSegElems) / kVecElems);
        w.sr = SCATTER ? w.t : source_row<GATHER>(ga, w.t);
        return w;
    };
    // the unit's elements into v (sr < 0: the registers are left as they
    // are).  Rows are streamed once (nontemporal); gathered source rows are
    // shared by the slots of a token and keep ordinary loads.
    auto load_unit = [&](const Unit& w, uint4 (&v)[NC]) {
        if (w.sr < 0) return;
        const uint4* xr = reinterpret_cast<const uint4*>(x + w.sr * K + w.e0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int idx = c * kWave + lane;
            if (idx < w.nvec) v[c] = GATHER ? xr[idx] : load_stream16(xr + idx);
            else v[c] = make_uint4(0, 0, 0, 0);
        }
    };

    uint4 v[NC], vn[NC];
    // the unit bookkeeping is wave-uniform: scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    int64_t u = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    Unit cu = unit(u);
    load_unit(cu, v);
    for (; u < units; u += nw) {
        const Unit nu = unit(u + nw);
        load_unit(nu, vn);
        const int64_t t = cu.t;
        const int nvec = cu.nvec;
        if constexpr (SCATTER) {
            // lane k < top_k holds the routed row of the token's slot k
            const int32_t my_row = lane < sc.top_k ? sc.ros[t * sc.top_k + lane] : -1;
            auto dest = [&](int k) {  // wave-uniform: the routed row of slot k, or -1
                const int32_t r = __builtin_amdgcn_readlane(my_row, k);
                return (r >= 0 && (int64_t)r < T && wave_row_covered(s_off, G, T, r)) ? (int64_t)r : (int64_t)-1;
            };
            if constexpr (FMT == 0) {
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
                const double inv = amax == 0.0f ? 0.0 : 1.0 / (double)scale;
                uint2 pk[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    float f[8];
                    unpack8(v[c], f);
                    if (amax != 0.0f) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) f[i] = div_by_scale(f[i], inv);
                    }
                    pk[c] = pack8_e4m3(f);
                }
                for (int k = 0; k < sc.top_k; ++k) {
                    const int64_t r = dest(k);
                    if (r < 0) continue;
                    uint8_t* qr = q + r * K;
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const int idx = c * kWave + lane;
                        if (idx < nvec) *reinterpret_cast<uint2*>(qr + (int64_t)idx * 8) = pk[c];
                    }
                    if (lane == 0) static_cast<float*>(scales)[r] = amax == 0.0f ? 0.0f : scale;
                }
            } else {
                constexpr bool FP4 = FMT == 2;
                uint2 pk[NC];
                int xs[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    float f[8];
                    unpack8(v[c], f);
                    xs[c] = mx_encode8<FP4>(f, pk[c]);
                }
                for (int k = 0; k < sc.top_k; ++k) {
                    const int64_t r = dest(k);
                    if (r < 0) continue;
                    uint8_t* qrow = q + r * (FP4 ? K / 2 : K) + (FP4 ? cu.e0 / 2 : cu.e0);
                    uint8_t* srow = static_cast<uint8_t*>(scales) + r * (K / 32) + cu.e0 / 32;
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const int idx = c * kWave + lane;
                        if (idx < nvec) mx_store8<FP4>(pk[c], xs[c], qrow, srow, idx, lane);
                    }
                }
            }
        } else if constexpr (FMT == 3) {
            const int g = cu.sr >= 0 ? wave_row_group(s_off, nv.ids, G, nv.E, T, t) : -1;
            // scale row: t, or in a padded layout the group's slot row (-1: past the tensor)
            int64_t srix = g >= 0 ? t : -1;
            if (g >= 0 && pd.soff) {
                const int64_t lo = (int64_t)s_off[g] < T ? (int64_t)s_off[g] : T;
                srix = (int64_t)pd.soff[g] + (t - lo);
                if (srix >= pd.S) srix = -1;
            }
            if (srix >= 0) {
                const float sf = nv.sf[nv.ids[g]];
                uint8_t* qrow = q + t * (K / 2) + cu.e0 / 2;
                uint8_t* srow = static_cast<uint8_t*>(scales) + srix * (K / 16) + cu.e0 / 16;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int idx = c * kWave + lane;
                    // a block's 2 lanes are both in or both out (K a multiple of 16)
                    float f[8];
                    unpack8(v[c], f);
                    uint32_t sc;
                    const uint32_t packed = nv_encode8(f, sf, sc);
                    if (idx < nvec) {
                        *reinterpret_cast<uint32_t*>(qrow + (int64_t)idx * 4) = packed;
                        if ((lane & 1) == 0) srow[idx >> 1] = (uint8_t)sc;
                    }
                }
            }
        } else if (cu.sr >= 0) {
            const int64_t srix = scale_row(pd, s_off, G, T, t);  // -1: the row is not written
            if (srix < 0) {
                // skipped (uncovered, or no scale row in the padded layout)
            } else if constexpr (FMT == 0) {
                // bf16 magnitudes order like their bit patterns with the sign cleared
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
                const double inv = amax == 0.0f ? 0.0 : 1.0 / (double)scale;
                uint8_t* qr = q + t * K;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int idx = c * kWave + lane;
                    if (idx >= nvec) continue;
                    float f[8];
                    unpack8(v[c], f);
                    // a zero row keeps its signed zeros (the convert keeps the sign)
                    if (amax != 0.0f) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) f[i] = div_by_scale(f[i], inv);
                    }
                    *reinterpret_cast<uint2*>(qr + (int64_t)idx * 8) = pack8_e4m3(f);
                }
                if (lane == 0) static_cast<float*>(scales)[t] = amax == 0.0f ? 0.0f : scale;
            } else {
                constexpr bool FP4 = FMT == 2;
                uint8_t* qrow = q + t * (FP4 ? K / 2 : K) + (FP4 ? cu.e0 / 2 : cu.e0);
                uint8_t* srow = static_cast<uint8_t*>(scales) + srix * (K / 32) + cu.e0 / 32;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int idx = c * kWave + lane;
                    // a block's 4 lanes are all in or all out (K is a multiple
                    // of 32), so the shuffles only mix lanes of one block
                    float f[8];
                    unpack8(v[c], f);
                    uint2 packed;
                    const int X = mx_encode8<FP4>(f, packed);
                    if (idx < nvec) mx_store8<FP4>(packed, X, qrow, srow, idx, lane);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) v[c] = vn[c];
        cu = nu;
    }
}

// FP8 rowwise rows longer than the register budget: the row is read twice,
// the amax pass and then the encode pass (from cache).  (MX and NVFP4 rows of
// any length are split into register-sized segments above.)
template <bool GATHER>
__global__ __launch_bounds__(kThreads) void quantize_long_kernel(const uint16_t* __restrict__ x,
                                                                 uint8_t* __restrict__ q, void* __restrict__ scales,
                                                                 const uint32_t* __restrict__ off, int G,
                                                                 int64_t T, int64_t K, Gather ga, Pad pd) {
    __shared__ uint32_t s_off[kMaxGroups + 1];
    load_offsets(s_off, off, G);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int64_t nvec = K / kVecElems;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; t < T; t += nw) {
        const int64_t sr = source_row<GATHER>(ga, t);
        if (sr < 0) continue;
        const uint4* xr = reinterpret_cast<const uint4*>(x + sr * K);
        if (scale_row(pd, s_off, G, T, t) < 0) continue;
        uint32_t amax_bits = 0;
        for (int64_t idx = lane; idx < nvec; idx += kWave) {
            const uint4 v = xr[idx];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int i = 0; i < 4; ++i) {
                amax_bits = max(amax_bits, w[i] & 0x7fffu);
                amax_bits = max(amax_bits, (w[i] >> 16) & 0x7fffu);
            }
        }
        const float amax = wave_max(bf16_to_f32(amax_bits));
        const float scale = amax / 448.0f;
        const double inv = amax == 0.0f ? 0.0 : 1.0 / (double)scale;
        uint8_t* qr = q + t * K;
        for (int64_t idx = lane; idx < nvec; idx += kWave) {
            float f[8];
            unpack8(load_stream16(xr + idx), f);
            if (amax != 0.0f)
                for (int i = 0; i < 8; ++i) f[i] = div_by_scale(f[i], inv);
            *reinterpret_cast<uint2*>(qr + idx * 8) = pack8_e4m3(f);
        }
        if (lane == 0) static_cast<float*>(scales)[t] = amax == 0.0f ? 0.0f : scale;
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
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int64_t nunits = I / 8;  // 8 outputs per lane-unit
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; t < T; t += nw) {
        if (!wave_row_covered(s_off, G, T, t)) continue;
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
            uint2 packed;
            const int X = mx_encode8<true>(y, packed);
            if (idx < nunits) mx_store8<true>(packed, X, qrow, srow, idx, lane);
        }
    }
}

// SwiGLU + NVFP4 requant: as above, with lane pairs forming 16-output blocks
// and the row's group supplying the expert's tensor scale of y.
__global__ __launch_bounds__(kThreads) void silu_quantize_nv_kernel(const uint16_t* __restrict__ h,
                                                                    uint8_t* __restrict__ yq,
                                                                    uint8_t* __restrict__ ys,
                                                                    const uint32_t* __restrict__ off, int G,
                                                                    int64_t T, int64_t I, NvScales nv) {
    __shared__ uint32_t s_off[kMaxGroups + 1];
    load_offsets(s_off, off, G);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = (int64_t)gridDim.x * kWavesPerBlock;
    const int64_t nunits = I / 8;  // even: I is a multiple of 16
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; t < T; t += nw) {
        const int g = wave_row_group(s_off, nv.ids, G, nv.E, T, t);
        if (g < 0) continue;
        const float sf = nv.sf[nv.ids[g]];
        const uint4* hr = reinterpret_cast<const uint4*>(h + t * 2 * I);
        uint8_t* qrow = yq + t * (I / 2);
        uint8_t* srow = ys + t * (I / 16);
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
            uint32_t sc;
            const uint32_t packed = nv_encode8(y, sf, sc);
            if (idx < nunits) {
                *reinterpret_cast<uint32_t*>(qrow + idx * 4) = packed;
                if ((lane & 1) == 0) srow[idx >> 1] = (uint8_t)sc;
            }
        }
    }
}

// Persistent grid: as many blocks as can be resident, at most one wave per
// work unit (row, or row segment).  The resident count of each kernel is
// asked of the runtime once per device and thread rather than at every
// launch.
template <auto KERNEL>
int64_t persistent_grid(int64_t units) {
    static thread_local int cached_dev = -1;
    static thread_local int64_t cached_cap = 0;
    int dev = 0;
    int64_t cap = 2048;
    if (hipGetDevice(&dev) == hipSuccess) {
        if (dev != cached_dev) {
            int cus = 0, occ = 0;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, KERNEL, kThreads, 0) == hipSuccess && cus > 0) {
                cached_cap = (int64_t)cus * (occ > 0 ? occ : 1);
                cached_dev = dev;
            }
        }
        if (dev == cached_dev) cap = cached_cap;
    }
    const int64_t need = (units + kWavesPerBlock - 1) / kWavesPerBlock;
    return need < cap ? need : cap;
}

// The register-resident kernel with NC chunks per unit: whole rows for FP8
// rowwise (K <= NC * 512), segments of NC * 512 elements for the block formats.
template <int FMT, int NC, bool GATHER, bool SCATTER>
hipError_t launch_rows(const uint16_t* x, uint8_t* q, void* s, const uint32_t* off, int G, int64_t T, int64_t K,
                       const Gather& ga, const NvScales& nv, const Pad& pd, const Scatter& sc, hipStream_t stream) {
    constexpr int64_t kSeg = (int64_t)NC * kChunk;
    const int64_t nseg = FMT == 0 ? 1 : (K + kSeg - 1) / kSeg;
    auto kernel = quantize_rows_kernel<FMT, NC, GATHER, SCATTER>;
    const int64_t rows = SCATTER ? sc.ntok : T;
    const int64_t grid = persistent_grid<quantize_rows_kernel<FMT, NC, GATHER, SCATTER>>(rows * nseg);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, q,
                       s, off, G, T, K, (int)nseg, ga, nv, pd, sc);
    return hipGetLastError();
}

template <int FMT, bool GATHER, bool SCATTER = false>
hipError_t launch_fmt(const uint16_t* x, uint8_t* q, void* s, const uint32_t* off, int G, int64_t T, int64_t K,
                      const Gather& ga, hipStream_t stream, const NvScales& nv = NvScales{nullptr, nullptr, 0},
                      const Pad& pd = Pad{nullptr, 0}, const Scatter& sc = Scatter{nullptr, 0, 0}) {
    const int64_t nc = (K + kChunk - 1) / kChunk;  // 512-element chunks per row
    if constexpr (FMT != 0) {
        // block formats: the fewest segments of at most 8 chunks, evened out
        const int64_t nseg = (nc + 7) / 8;
        const int64_t per = (nc + nseg - 1) / nseg;
        if (per <= 1) return launch_rows<FMT, 1, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if (per <= 2) return launch_rows<FMT, 2, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if (per <= 4) return launch_rows<FMT, 4, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if (per <= 7) return launch_rows<FMT, 7, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        return launch_rows<FMT, 8, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
    } else {
        if (nc <= 1) return launch_rows<FMT, 1, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if (nc <= 2) return launch_rows<FMT, 2, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if (nc <= 4) return launch_rows<FMT, 4, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if (nc <= 8) return launch_rows<FMT, 8, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if (nc <= 14) return launch_rows<FMT, 14, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if (nc <= 16) return launch_rows<FMT, 16, GATHER, SCATTER>(x, q, s, off, G, T, K, ga, nv, pd, sc, stream);
        if constexpr (SCATTER) {
            return hipErrorInvalidValue;  // token rows past 8192 elements (refused by the C ABI before this)
        } else {
            auto kernel = quantize_long_kernel<GATHER>;
            hipLaunchKernelGGL(kernel, dim3((unsigned)persistent_grid<quantize_long_kernel<GATHER>>(T)), dim3(kThreads),
                               0, stream, x, q, s,
                               off, G, T, K, ga, pd);
            return hipGetLastError();
        }
    }
}

template <bool GATHER>
hipError_t launch_any(int fmt, const void* x, void* q, void* scales, const uint32_t* off, int G, int64_t T,
                      int64_t K, const Gather& ga, hipStream_t stream) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint8_t* qb = static_cast<uint8_t*>(q);
    if (fmt == 0) return launch_fmt<0, GATHER>(xb, qb, scales, off, G, T, K, ga, stream);
    if (fmt == 1) return launch_fmt<1, GATHER>(xb, qb, scales, off, G, T, K, ga, stream);
    return launch_fmt<2, GATHER>(xb, qb, scales, off, G, T, K, ga, stream);
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_quantize(int fmt, const void* x, void* q, void* scales, const uint32_t* off, int G, int64_t T,
                           int64_t K, hipStream_t stream) {
    return launch_any<false>(fmt, x, q, scales, off, G, T, K, Gather{nullptr, 1, T}, stream);
}

hipError_t launch_quantize_gather(int fmt, const void* x, int64_t nsrc, const int32_t* indices, int32_t divisor,
                                  void* q, void* scales, const uint32_t* off, int G, int64_t T, int64_t K,
                                  hipStream_t stream) {
    return launch_any<true>(fmt, x, q, scales, off, G, T, K, Gather{indices, divisor, nsrc}, stream);
}

hipError_t launch_quantize_scatter(int fmt, const void* x, int64_t ntok, const int32_t* row_of_slot, int top_k,
                                   void* q, void* scales, const uint32_t* off, int G, int64_t T, int64_t K,
                                   hipStream_t stream) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint8_t* qb = static_cast<uint8_t*>(q);
    const Gather ga{nullptr, 1, ntok};
    const NvScales nv{nullptr, nullptr, 0};
    const Pad pd{nullptr, 0};
    const Scatter sc{row_of_slot, top_k, ntok};
    if (fmt == 0) return launch_fmt<0, false, true>(xb, qb, scales, off, G, T, K, ga, stream, nv, pd, sc);
    if (fmt == 1) return launch_fmt<1, false, true>(xb, qb, scales, off, G, T, K, ga, stream, nv, pd, sc);
    return launch_fmt<2, false, true>(xb, qb, scales, off, G, T, K, ga, stream, nv, pd, sc);
}

hipError_t launch_quantize_padded(int fmt, const void* x, void* q, void* scales, const uint32_t* scales_offsets,
                                  int64_t scale_rows, const uint32_t* off, int G, int64_t T, int64_t K,
                                  hipStream_t stream) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint8_t* qb = static_cast<uint8_t*>(q);
    const Gather ga{nullptr, 1, T};
    const NvScales nv{nullptr, nullptr, 0};
    const Pad pd{scales_offsets, scale_rows};
    if (fmt == 1) return launch_fmt<1, false>(xb, qb, scales, off, G, T, K, ga, stream, nv, pd);
    return launch_fmt<2, false>(xb, qb, scales, off, G, T, K, ga, stream, nv, pd);
}

hipError_t launch_quantize_nvfp4(const void* x, void* q, void* scales, const float* tensor_scales,
                                  const uint32_t* off, const int32_t* ids, int G, int E, int64_t T, int64_t K,
                                  hipStream_t stream) {
    return launch_fmt<3, false>(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), scales, off, G, T, K,
                                Gather{nullptr, 1, T}, stream, NvScales{ids, tensor_scales, E});
}

hipError_t launch_quantize_nvfp4_padded(const void* x, void* q, void* scales, const float* tensor_scales,
                                        const uint32_t* scales_offsets, int64_t scale_rows, const uint32_t* off,
                                        const int32_t* ids, int G, int E, int64_t T, int64_t K, hipStream_t stream) {
    return launch_fmt<3, false>(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(q), scales, off, G, T, K,
                                Gather{nullptr, 1, T}, stream, NvScales{ids, tensor_scales, E},
                                Pad{scales_offsets, scale_rows});
}

hipError_t launch_silu_quantize(const void* h, void* yq, void* ys, const uint32_t* off, int G, int64_t T,
                                int64_t I, hipStream_t stream) {
    hipLaunchKernelGGL(silu_quantize_kernel, dim3((unsigned)persistent_grid<silu_quantize_kernel>(T)), dim3(kThreads),
                       0, stream, static_cast<const uint16_t*>(h), static_cast<uint8_t*>(yq), static_cast<uint8_t*>(ys),
                       off, G, T, I);
    return hipGetLastError();
}

hipError_t launch_silu_quantize_nvfp4(const void* h, void* yq, void* ys, const float* y_sf, const uint32_t* off,
                                      const int32_t* ids, int G, int E, int64_t T, int64_t I, hipStream_t stream) {
    hipLaunchKernelGGL(silu_quantize_nv_kernel, dim3((unsigned)persistent_grid<silu_quantize_nv_kernel>(T)),
                       dim3(kThreads), 0, stream, static_cast<const uint16_t*>(h), static_cast<uint8_t*>(yq),
                       static_cast<uint8_t*>(ys), off, G, T, I, NvScales{ids, y_sf, E});
    return hipGetLastError();
}

}  // namespace mxg
