// gemm.hip -- ragged grouped GEMM for gfx950 (FP8 rowwise, MXFP8, MXFP4), with
// a BF16 epilogue or the fused SwiGLU + MXFP4 requant epilogue.
//
// (grouped_matmul_rowwise_dynamic_scaled_fp8, description: out[t,n] =
//  (sum_k a[t,k] b[expert_ids[g],n,k]) a_scale[t] b_scale[expert_ids[g],n],
//  fp32 accumulation, one post-reduction scale; NvMxf4f8Strategy,
//  grouped_matmul() and grouped_matmul_swiglu().)
//
// Design (CDNA4):
//  * Matrix core: v_mfma_scale_f32_32x32x64_f8f6f4.  Lane l (h = l / 32)
//    holds row l % 32 of A (or column of B) for one 64-deep K step, and lane
//    r + 32*b supplies the E8M0 scale of block b (K 32b .. 32b+31) of row r.
//    Operand bytes map to K differently per element width (measured on
//    gfx950 with single-element probes):
//      e2m1: the 32 nibbles of lane half h are K 32h .. 32h+31 (low nibble
//            first), i.e. all of block h;
//      e4m3: bytes 0..15 are K 16h .. 16h+15 (block 0) and bytes 16..31 are
//            K 32+16h .. 32+16h+15 (block 1).
//    FP8 rowwise runs the same instruction without block scales and applies
//    a_scale * b_scale in the epilogue.
//  * Tiles: a workgroup of 4 waves (2 x 2) owns a BM x BN output tile; each
//    wave a (BM/2) x (BN/2) sub-tile of 32 x 32 accumulators.  K streams in
//    stages of 128 bytes per row (128 e4m3 or 256 e2m1 elements) through a
//    double-buffered LDS ring: global -> registers for stage k+1 is in flight
//    while stage k feeds the matrix cores.  16-byte chunks are XOR-swizzled by
//    row so the 16-byte LDS reads of 8 consecutive rows hit distinct banks.
//  * Ragged groups without host sync: every workgroup derives the per-group
//    M-tile counts from row_offsets into an LDS prefix sum; a tile index is
//    mapped to (group, m-tile) by binary search.  Empty or invalid groups own
//    no tiles, partial M tiles are masked, not padded in memory.
//  * Persistent, XCD-aware schedule: the grid is sized to the resident
//    capacity; workgroup b (dispatched to XCD b % 8) walks logical tiles so
//    that the workgroups resident on one XCD hold consecutive tiles (same
//    expert, neighbouring N tiles), which keeps shared A/B panels in that
//    XCD's L2.
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kStageBytes = 128;  // K bytes per row per stage
constexpr int kNumXcd = 8;

struct GemmArgs {
    const uint8_t* a;
    const void* as;
    const uint8_t* b;
    const void* bs;
    uint16_t* c;
    uint8_t* yq;
    uint8_t* ys;
    const uint32_t* off;
    const int32_t* ids;
    int G;
    int E;
    int64_t T;
    int64_t N;
    int64_t K;
    int64_t row_bytes;  // bytes per row of a and b
    int ntiles_n;
};

// FMT: 0 = FP8 rowwise, 1 = MXFP8, 2 = MXFP4.
template <int FMT>
struct Fmt {
    static constexpr bool kMX = FMT != 0;
    static constexpr bool kFP4 = FMT == 2;
    static constexpr int kSteps = kFP4 ? 4 : 2;           // 64-deep MFMA steps per stage
    static constexpr int kBlocks = kFP4 ? 8 : 4;          // 32-element scale blocks per stage
    static constexpr int kTypeCode = kFP4 ? 4 : 0;        // cbsz / blgp: 0 = e4m3, 4 = e2m1
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kStageBytes + ((chunk ^ (row & 7)) << 4); }

// Bijective remap so that the workgroups the dispatcher sends to one XCD
// (b, b + 8, b + 16, ...) get consecutive logical indices.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int per = n / kNumXcd, rem = n % kNumXcd;
    const int xcd = b % kNumXcd, idx = b / kNumXcd;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Exclusive block-wide scan (256 threads).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t n = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += n;
    }
    if (lane == kWave - 1) s_wave[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
        uint32_t s = s_wave[w];
        before += w < wave ? s : 0;
        all += s;
    }
    *total = all;
    return before + inc - v;
}

template <int BM, int BN, int FMT, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(const GemmArgs args) {
    using F = Fmt<FMT>;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int A_CH = BM * 8 / kThreads;  // 16-byte chunks per thread per stage
    constexpr int B_CH = BN * 8 / kThreads;
    constexpr int A_SC = F::kMX ? BM * F::kBlocks / kThreads : 0;  // scale bytes per thread per stage
    constexpr int B_SC = F::kMX ? BN * F::kBlocks / kThreads : 0;
    static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for the loader");
    static_assert(!F::kMX || (A_SC >= 1 && B_SC >= 1), "tile too small for the scale loader");
    constexpr int kAStage = BM * kStageBytes, kBStage = BN * kStageBytes;
    constexpr int kSStride = 8;  // LDS bytes per row of a stage's scales

    __shared__ __attribute__((aligned(16))) uint8_t s_ab[2 * (kAStage + kBStage)];
    __shared__ uint8_t s_sc[F::kMX ? 2 * (BM + BN) * kSStride : 4];
    __shared__ uint32_t s_pre[kMaxGroups + 1];
    __shared__ uint32_t s_wave[kThreads / kWave];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int G = args.G;

    // ---- per-group M-tile prefix (ragged schedule, no host sync)
    {
        uint32_t cnt[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = tid * 4 + i;
            cnt[i] = 0;
            if (g < G) {
                GroupRange r = group_range(args.off, args.ids, g, args.T, args.E);
                cnt[i] = (uint32_t)((r.hi - r.lo + BM - 1) / BM);
            }
            local += cnt[i];
        }
        uint32_t total;
        uint32_t ex = block_exclusive_scan(local, s_wave, &total);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = tid * 4 + i;
            if (g < G) s_pre[g] = ex;
            ex += cnt[i];
        }
        if (tid == 0) s_pre[G] = total;
        __syncthreads();
    }
    const int64_t total_tiles = (int64_t)s_pre[G] * args.ntiles_n;
    const int nkt = (int)((args.row_bytes + kStageBytes - 1) / kStageBytes);

    for (int64_t L = xcd_remap(blockIdx.x, gridDim.x); L < total_tiles; L += gridDim.x) {
        const int mt = (int)(L / args.ntiles_n);
        const int nt = (int)(L % args.ntiles_n);
        // group owning m-tile mt: largest g with s_pre[g] <= mt
        int lo = 0, hi = G;  // invariant: s_pre[lo] <= mt < s_pre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_pre[mid] <= (uint32_t)mt) lo = mid; else hi = mid;
        }
        const int g = lo;
        const GroupRange gr = group_range(args.off, args.ids, g, args.T, args.E);
        const int e = args.ids[g];
        const int64_t m0 = gr.lo + (int64_t)(mt - (int)s_pre[g]) * BM;
        const int64_t m_end = m0 + BM < gr.hi ? m0 + BM : gr.hi;
        const int64_t n0 = (int64_t)nt * BN;

        // ---- global load plan for this tile
        const uint8_t* a_row[A_CH];
        const uint8_t* b_row[B_CH];
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int q = tid + kThreads * i, r = q >> 3;
            int64_t row = m0 + r;
            row = row < m_end ? row : m_end - 1;
            a_row[i] = args.a + row * args.row_bytes + ((q & 7) << 4);
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int q = tid + kThreads * i, r = q >> 3;
            int64_t n = n0 + r;
            n = n < args.N ? n : args.N - 1;
            b_row[i] = args.b + ((int64_t)e * args.N + n) * args.row_bytes + ((q & 7) << 4);
        }
        uint4 ra[A_CH], rb[B_CH];
        uint8_t rsa[A_SC > 0 ? A_SC : 1], rsb[B_SC > 0 ? B_SC : 1];

        auto load_stage = [&](int kt) {
            const int64_t kb = (int64_t)kt * kStageBytes;
#pragma unroll
            for (int i = 0; i < A_CH; ++i) {
                const int c = (tid + kThreads * i) & 7;
                ra[i] = kb + c * 16 < args.row_bytes ? *reinterpret_cast<const uint4*>(a_row[i] + kb)
                                                     : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const int c = (tid + kThreads * i) & 7;
                rb[i] = kb + c * 16 < args.row_bytes ? *reinterpret_cast<const uint4*>(b_row[i] + kb)
                                                     : make_uint4(0, 0, 0, 0);
            }
            if constexpr (F::kMX) {
                const int64_t nblk = args.K / 32;
                const uint8_t* as = static_cast<const uint8_t*>(args.as);
                const uint8_t* bs = static_cast<const uint8_t*>(args.bs);
#pragma unroll
                for (int i = 0; i < A_SC; ++i) {
                    const int q = tid + kThreads * i, r = q / F::kBlocks, j = q % F::kBlocks;
                    int64_t row = m0 + r;
                    row = row < m_end ? row : m_end - 1;
                    const int64_t blk = (int64_t)kt * F::kBlocks + j;
                    rsa[i] = blk < nblk ? as[row * nblk + blk] : (uint8_t)127;
                }
#pragma unroll
                for (int i = 0; i < B_SC; ++i) {
                    const int q = tid + kThreads * i, r = q / F::kBlocks, j = q % F::kBlocks;
                    int64_t n = n0 + r;
                    n = n < args.N ? n : args.N - 1;
                    const int64_t blk = (int64_t)kt * F::kBlocks + j;
                    rsb[i] = blk < nblk ? bs[((int64_t)e * args.N + n) * nblk + blk] : (uint8_t)127;
                }
            }
        };
        auto store_stage = [&](int st) {
            uint8_t* sa = s_ab + st * (kAStage + kBStage);
            uint8_t* sb = sa + kAStage;
#pragma unroll
            for (int i = 0; i < A_CH; ++i) {
                const int q = tid + kThreads * i;
                *reinterpret_cast<uint4*>(sa + swz(q >> 3, q & 7)) = ra[i];
            }
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const int q = tid + kThreads * i;
                *reinterpret_cast<uint4*>(sb + swz(q >> 3, q & 7)) = rb[i];
            }
            if constexpr (F::kMX) {
                uint8_t* ssa = s_sc + st * (BM + BN) * kSStride;
                uint8_t* ssb = ssa + BM * kSStride;
#pragma unroll
                for (int i = 0; i < A_SC; ++i) {
                    const int q = tid + kThreads * i;
                    ssa[(q / F::kBlocks) * kSStride + q % F::kBlocks] = rsa[i];
                }
#pragma unroll
                for (int i = 0; i < B_SC; ++i) {
                    const int q = tid + kThreads * i;
                    ssb[(q / F::kBlocks) * kSStride + q % F::kBlocks] = rsb[i];
                }
            }
        };

        v16f acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};

        load_stage(0);
        store_stage(0);
        __syncthreads();

        const int h = lane >> 5, r32 = lane & 31;
        for (int kt = 0; kt < nkt; ++kt) {
            const int st = kt & 1;
            if (kt + 1 < nkt) load_stage(kt + 1);
            const uint8_t* sa = s_ab + st * (kAStage + kBStage);
            const uint8_t* sb = sa + kAStage;
            const uint8_t* ssa = s_sc + st * (BM + BN) * kSStride;
            const uint8_t* ssb = ssa + BM * kSStride;
#pragma unroll
            for (int s = 0; s < F::kSteps; ++s) {
                v8i af[TM], bf[TN];
                int sca[TM], scb[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int row = wm * WM + i * 32 + r32;
                    if constexpr (F::kFP4) {
                        const uint4 x = *reinterpret_cast<const uint4*>(sa + swz(row, 2 * s + h));
                        af[i] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
                    } else {
                        const uint4 x0 = *reinterpret_cast<const uint4*>(sa + swz(row, 4 * s + h));
                        const uint4 x1 = *reinterpret_cast<const uint4*>(sa + swz(row, 4 * s + 2 + h));
                        af[i] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                    (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                    }
                    if constexpr (F::kMX) sca[i] = ssa[row * kSStride + 2 * s + h];
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int row = wn * WN + j * 32 + r32;
                    if constexpr (F::kFP4) {
                        const uint4 x = *reinterpret_cast<const uint4*>(sb + swz(row, 2 * s + h));
                        bf[j] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
                    } else {
                        const uint4 x0 = *reinterpret_cast<const uint4*>(sb + swz(row, 4 * s + h));
                        const uint4 x1 = *reinterpret_cast<const uint4*>(sb + swz(row, 4 * s + 2 + h));
                        bf[j] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                    (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                    }
                    if constexpr (F::kMX) scb[j] = ssb[row * kSStride + 2 * s + h];
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        if constexpr (F::kMX)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                af[i], bf[j], acc[i][j], F::kTypeCode, F::kTypeCode, 0, sca[i], 0, scb[j]);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                af[i], bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
                    }
            }
            if (kt + 1 < nkt) store_stage(st ^ 1);
            __syncthreads();
        }

        // ---- epilogue
        if constexpr (!SWIGLU) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t col = n0 + wn * WN + j * 32 + r32;
                    float sbv = 1.0f;
                    if constexpr (!F::kMX)
                        if (col < args.N) sbv = static_cast<const float*>(args.bs)[(int64_t)e * args.N + col];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (row < m_end && col < args.N) {
                            float v = acc[i][j][r];
                            if constexpr (!F::kMX) {
                                v = v * static_cast<const float*>(args.as)[row];
                                v = v * sbv;
                            }
                            args.c[row * args.N + col] = (uint16_t)f32_to_bf16(v);
                        }
                    }
                }
        } else {
            // Stage the bf16 gate/up tile in LDS, then requant rows of 32 outputs
            // with the same code the standalone activation kernel runs.
            static_assert(BN % 64 == 0, "fused tile must hold whole 32-output blocks");
            static_assert(BM * BN * 2 <= 2 * (kAStage + kBStage), "staging tile must fit the LDS ring");
            uint16_t* s_c = reinterpret_cast<uint16_t*>(s_ab);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = wn * WN + j * 32 + r32;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        s_c[row * BN + col] = (uint16_t)f32_to_bf16(acc[i][j][r]);
                    }
                }
            __syncthreads();
            constexpr int kBlk = BN / 64;  // 32-output blocks per tile row
            constexpr int kUnits = BM * kBlk;
            const int l4 = tid & 3;
            const int64_t I = args.N / 2;
#pragma unroll 1
            for (int u = tid >> 2; u < kUnits; u += kThreads / 4) {
                const int row = u / kBlk, blk = u % kBlk;
                const uint4* src = reinterpret_cast<const uint4*>(s_c + row * BN + blk * 64 + l4 * 16);
                float gu[16];
                unpack8(src[0], gu);
                unpack8(src[1], gu + 8);
                float y[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = bf16_to_f32(f32_to_bf16(silu_mul(gu[2 * k], gu[2 * k + 1])));
                uint32_t code[8];
                const int X = mx_encode8<true>(y, code);
                const int64_t grow = m0 + row;
                const int64_t gblk = n0 / 64 + blk;
                if (grow < m_end && n0 + blk * 64 < args.N) {
                    // unit index within the output row, in 8-output lane units
                    mx_store8<true>(code, X, args.yq + grow * (I / 2), args.ys + grow * (I / 32), gblk * 4 + l4, l4);
                }
            }
        }
        __syncthreads();  // LDS is reused by the next tile's prologue
    }
}

// ---------------------------------------------------------------------------
struct LaunchCache {
    int device = -1;
    int cus = 0;
};

int device_cus() {
    static thread_local LaunchCache cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (cache.device != dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache.device = dev;
        cache.cus = cus;
    }
    return cache.cus;
}

template <int BM, int BN, int FMT, bool SWIGLU>
hipError_t launch_tile(const GemmProblem& p, hipStream_t stream) {
    auto kernel = grouped_gemm_kernel<BM, BN, FMT, SWIGLU>;
    static thread_local int occ_device = -1, occ = 0;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (occ_device != dev) {
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0);
        if (err != hipSuccess) return err;
        occ_device = dev;
    }
    const int cus = device_cus();
    GemmArgs a;
    a.a = static_cast<const uint8_t*>(p.a);
    a.as = p.a_scales;
    a.b = static_cast<const uint8_t*>(p.b);
    a.bs = p.b_scales;
    a.c = static_cast<uint16_t*>(p.c);
    a.yq = static_cast<uint8_t*>(p.yq);
    a.ys = static_cast<uint8_t*>(p.ys);
    a.off = p.off;
    a.ids = p.ids;
    a.G = p.G;
    a.E = p.E;
    a.T = p.T;
    a.N = p.N;
    a.K = p.K;
    a.row_bytes = FMT == 2 ? p.K / 2 : p.K;
    a.ntiles_n = (int)((p.N + BN - 1) / BN);
    // Upper bound on M tiles: each non-empty group adds at most one partial tile.
    const int64_t groups_nonempty = p.G < p.T ? p.G : p.T;
    const int64_t mtiles_bound = p.T / BM + groups_nonempty;
    const int64_t tiles_bound = mtiles_bound * a.ntiles_n;
    int64_t grid = (int64_t)(cus > 0 ? cus : 256) * (occ > 0 ? occ : 1);
    if (grid > tiles_bound) grid = tiles_bound;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream) {
    const bool swiglu = p.yq != nullptr;
    switch (p.fmt) {
        case 0:
            return launch_tile<128, 128, 0, false>(p, stream);
        case 1:
            return swiglu ? launch_tile<128, 128, 1, true>(p, stream) : launch_tile<128, 128, 1, false>(p, stream);
        case 2:
            return swiglu ? launch_tile<128, 128, 2, true>(p, stream) : launch_tile<128, 128, 2, false>(p, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace mxg
