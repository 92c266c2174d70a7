// gemm_common.h -- pieces both grouped-GEMM kernels share: argument block,
// per-format constants, the LDS swizzle, the XCD-aware tile order, the ragged
// tile map (per-group M-tile prefix in LDS + binary search) and the counted
// wait / barrier primitives of the K pipeline.  Device code for gfx950.
#pragma once

#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace gemm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kStageBytes = 128;  // K bytes per row per stage (block formats; FP8 rowwise may use 64)
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
    int mband;          // tile order within a group: bands of mband M tiles, N walked within a band
                        // (1: M tiles outer; >= the group's M tiles: N tiles outer)
    const float* es;    // NVFP4: per-expert epilogue scale (fp32 [E]); unused otherwise
    const uint16_t* rs; // NVFP4 fused: optional bf16 scale per routed row (nullptr: 1)
    const float* ysf;   // NVFP4 fused: per-expert encode-side tensor scale of y (fp32 [E])
    const uint32_t* asoff;  // padded MX A scales: group g's rows start at scale row asoff[g] (nullptr: dense)
    int64_t as_rows;        // rows of the padded A scale tensor
};

// FMT: 0 = FP8 rowwise, 1 = MXFP8, 2 = MXFP4, 3 = NVFP4.
template <int FMT>
struct Fmt {
    static constexpr bool kMX = FMT != 0;          // block scales (E8M0, or E4M3 for NVFP4)
    static constexpr bool kNV = FMT == 3;          // 16-element blocks, E4M3 scales, f16 matrix cores
    static constexpr bool kFP4 = FMT == 2 || FMT == 3;
    static constexpr int kBlockElems = kNV ? 16 : 32;
    static constexpr int kBlocks = (kFP4 ? 256 : 128) / kBlockElems;  // scale blocks (bytes) per 128-byte stage
    static constexpr int kWords = kBlocks / 4;     // scale words per row per stage
    static constexpr int kTypeCode = kFP4 ? 4 : 0;  // cbsz / blgp: 0 = e4m3, 4 = e2m1
};

// LDS byte offset of 16-byte chunk `chunk` of stage row `row`, for stage rows
// of SB bytes (K bytes per row per stage: 128 or 64).  A ds_read_b128 serves
// 16 lanes at a time across the 64 four-byte banks (16 four-bank groups), and
// a fragment read's 16-lane slice reads one chunk of 16 consecutive rows.
//  * SB = 128: a row covers 8 groups, so even and odd rows fall in opposite
//    halves; XOR-ing the chunk with bits 1..3 of the row spreads the 16 rows
//    over 16 distinct groups.
//  * SB = 64: a row covers 4 groups, so rows r, r + 4, r + 8, r + 12 start in
//    the same group; XOR-ing the chunk with bits 2..3 of the row separates them.
template <int SB>
__device__ __forceinline__ int swz_chunk(int row, int chunk) {
    static_assert(SB == 128 || SB == 64, "stage rows of 128 or 64 bytes");
    return SB == 128 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 2) & 3);
}
template <int SB>
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * SB + (swz_chunk<SB>(row, chunk) << 4);
}

// Bijective remap so that the workgroups the dispatcher sends to one XCD
// (b, b + 8, b + 16, ...) get consecutive logical indices.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int per = n / kNumXcd, rem = n % kNumXcd;
    const int xcd = b % kNumXcd, idx = b / kNumXcd;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Exclusive block-wide scan over NT threads.
template <int NT>
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
    for (int w = 0; w < NT / kWave; ++w) {
        uint32_t s = s_wave[w];
        before += w < wave ? s : 0;
        all += s;
    }
    *total = all;
    return before + inc - v;
}

// Scale bytes p[0 .. 4) as one word; bytes at or past `avail` read as 127
// (2^0: they only ever multiply zero-filled K tails).
__device__ __forceinline__ uint32_t scale_word(const uint8_t* p, int64_t avail) {
    if (avail >= 4 && (reinterpret_cast<uintptr_t>(p) & 3) == 0) return *reinterpret_cast<const uint32_t*>(p);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= (uint32_t)(i < avail ? p[i] : (uint8_t)127) << (8 * i);
    return w;
}

// s_waitcnt vmcnt(N) (expcnt / lgkmcnt left at their maxima): wait until at
// most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the K loop.  __syncthreads() carries a workgroup
// release fence, and because direct-to-LDS loads count as LDS writes that
// fence waits for ALL of them (vmcnt(0)), draining the prefetch in flight.
// Here each wave waits only until at most N of its loads are outstanding
// (the stage being prefetched) and for its own LDS writes (lgkmcnt(0)); the
// empty asm statements keep the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    wait_vmem<N>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const void __attribute__((address_space(3)))*)p;
}

// A direct-to-LDS load, 16 bytes per lane (global_load_lds_dwordx4), issued
// from inline assembly for the rings of 64-byte stages.  The compiler then does not
// see an LDS write and adds no waits of its own before LDS reads (with the
// builtin, its alias tracking of the loads in flight gave up at the ring
// loop's head and drained them before every fourth stage); the ring's
// counted vmcnt waits and barriers order the reads instead, so such a K
// loop must issue no other vector-memory instruction.  base: wave-uniform
// global address; voff: this lane's byte offset from it; lds: wave-uniform
// LDS address of the 1 KiB the wave's 64 lanes fill (lane l at lds + 16 l).
// M0 carries the LDS address and is restored afterwards; the s_nop gives the
// M0 write and an SGPR operand written by a vector instruction just before
// their wait states.  Only the saved copy of M0 is written (by a scalar
// move, at once).
template <bool NT>
__device__ __forceinline__ void lds_dma16(const void* base_in, uint32_t voff, uint32_t lds_in) {
    // the operands are wave-uniform; read them from the first lane so that
    // they sit in scalar registers whatever the compiler can prove (the
    // builtin returns int: each half goes through uint32_t, so the low half
    // is not sign-extended into the high one)
    const uint64_t b = (uint64_t)base_in;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(lds_in);
    uint32_t saved_m0;
    if constexpr (NT)
        __asm__ volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\t"
            "global_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
            : "=&s"(saved_m0)
            : "v"(voff), "s"(base), "s"(lds)
            : "memory");
    else
        __asm__ volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\t"
            "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
            : "=&s"(saved_m0)
            : "v"(voff), "s"(base), "s"(lds)
            : "memory");
}

// Cache-policy operand of the direct global -> LDS load: the nontemporal bit
// (the line is marked to be replaced first; data still comes through L2).
constexpr int kCpolNT = 2;

// ---------------------------------------------------------------------------
// Ragged tile map.  Each workgroup turns row_offsets into a prefix over the
// per-group M-tile counts (in LDS; groups that are empty, inverted or carry an
// out-of-range expert id own no tiles).  Tile L of the launch is then found by
// binary search.  Within a group the tiles run in bands of mband M tiles
// with the N index outer inside a band, so the tiles in flight together on
// one XCD cover about mband M tiles by (tiles per XCD / mband) N tiles and
// share both A and weight panels in that XCD's L2 (mband = 1: M-outer;
// mband at least the group's M tiles: N-outer).
template <int NT, int BM>
__device__ __forceinline__ void build_tile_prefix(const GemmArgs& args, uint32_t* s_pre, uint32_t* s_wave) {
    constexpr int kPer = (kMaxGroups + NT - 1) / NT;
    const int tid = threadIdx.x, G = args.G;
    uint32_t cnt[kPer], local = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int g = tid * kPer + i;
        cnt[i] = 0;
        if (g < G) {
            const GroupRange r = group_range(args.off, args.ids, g, args.T, args.E);
            cnt[i] = (uint32_t)((r.hi - r.lo + BM - 1) / BM);
        }
        local += cnt[i];
    }
    uint32_t total;
    uint32_t ex = block_exclusive_scan<NT>(local, s_wave, &total);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int g = tid * kPer + i;
        if (g < G) s_pre[g] = ex;
        ex += cnt[i];
    }
    if (tid == 0) s_pre[G] = total;
    __syncthreads();
}

struct TileCoord {
    int g;           // group
    int64_t glo;     // the group's first row
    int e;           // expert
    int64_t m0;      // first row of the tile
    int64_t m_end;   // one past its last real row
    int64_t n0;      // first column
    int64_t n_end;   // one past its last real column
    int rows_in;     // real rows (1 .. BM)
    int cols_in;     // real columns (0 .. BN; 0: an empty half tile)
};

// Work items of a persistent launch.  When the tiles leave a last round
// that is at most half full, each of its R tiles is split into two half
// tiles along N (columns [n0, n0 + BN/2) and [n0 + BN/2, n0 + BN)): 2R items
// of about 3/4 of a tile's load time each fill the round better than R
// whole tiles.
struct WorkSplit {
    int64_t full;   // items before the split round (whole tiles)
    int64_t items;  // all items
};

__device__ __forceinline__ WorkSplit work_split(int64_t total_tiles, int64_t grid) {
    const int64_t rem = total_tiles % grid;
    WorkSplit w;
    w.full = total_tiles - rem;
    w.items = (rem > 0 && 2 * rem <= grid) ? w.full + 2 * rem : total_tiles;
    if (w.items == total_tiles) w.full = total_tiles;
    return w;
}

template <int BM, int BN>
__device__ __forceinline__ TileCoord locate_tile(const GemmArgs& args, const uint32_t* s_pre, int64_t L) {
    const int ntn = args.ntiles_n;
    int lo = 0, hi = args.G;  // invariant: s_pre[lo] * ntn <= L < s_pre[hi] * ntn
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)s_pre[mid] * ntn <= L) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int mtiles = (int)(s_pre[g + 1] - s_pre[g]);
    const int local = (int)(L - (int64_t)s_pre[g] * ntn);
    const int mb = args.mband < mtiles ? args.mband : mtiles;  // mb * ntn <= the group's tiles
    const int band = local / (mb * ntn);
    const int r = local - band * mb * ntn;
    const int left = mtiles - band * mb;
    const int gm = left < mb ? left : mb;  // M tiles in this band
    const int mt = band * mb + r % gm;
    const int nt = r / gm;
    const GroupRange gr = group_range(args.off, args.ids, g, args.T, args.E);
    TileCoord t;
    t.g = g;
    t.glo = gr.lo;
    t.e = args.ids[g];
    t.m0 = gr.lo + (int64_t)mt * BM;
    t.m_end = t.m0 + BM < gr.hi ? t.m0 + BM : gr.hi;
    t.n0 = (int64_t)nt * BN;
    t.rows_in = (int)(t.m_end - t.m0);
    t.cols_in = (int)(args.N - t.n0 < BN ? args.N - t.n0 : BN);
    t.n_end = t.n0 + t.cols_in;
    return t;
}

// The coordinates are the same in every lane (they derive from the launch
// arguments and the LDS prefix alone); read from the first lane, they sit in
// scalar registers instead of taking vector registers through the K loop.
__device__ __forceinline__ int64_t first_lane64(int64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}
__device__ __forceinline__ TileCoord uniform_coord(TileCoord t) {
    t.g = __builtin_amdgcn_readfirstlane(t.g);
    t.glo = first_lane64(t.glo);
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.m0 = first_lane64(t.m0);
    t.m_end = first_lane64(t.m_end);
    t.n0 = first_lane64(t.n0);
    t.n_end = first_lane64(t.n_end);
    t.rows_in = __builtin_amdgcn_readfirstlane(t.rows_in);
    t.cols_in = __builtin_amdgcn_readfirstlane(t.cols_in);
    return t;
}

// Item W of a launch split as work_split describes.
template <int BM, int BN>
__device__ __forceinline__ TileCoord locate_item(const GemmArgs& args, const uint32_t* s_pre, const WorkSplit& ws,
                                                 int64_t W) {
    if (W < ws.full) return locate_tile<BM, BN>(args, s_pre, W);
    TileCoord t = locate_tile<BM, BN>(args, s_pre, ws.full + (W - ws.full) / 2);
    const int half = (int)((W - ws.full) % 2);
    t.n0 += half * (BN / 2);
    const int64_t left = t.n_end - t.n0;
    t.cols_in = (int)(left < BN / 2 ? (left > 0 ? left : 0) : BN / 2);
    t.n_end = t.n0 + t.cols_in;
    return t;
}

// ---------------------------------------------------------------------------
// Host side.
int device_cus();

// Argument block for a BM x BN tiling of problem p; also returns the launch
// grid (resident capacity `per_cu` x CUs, capped by an upper bound on the
// tile count).  grid == 0 means there is nothing to do.
GemmArgs make_args(const GemmProblem& p, int BM, int BN, int mband, int per_cu, int64_t* grid);

}  // namespace gemm
}  // namespace mxg
