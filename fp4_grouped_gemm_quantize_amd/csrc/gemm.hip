// gemm.hip -- ragged grouped GEMM for gfx950 (FP8 rowwise, MXFP8, MXFP4), with
// a BF16 epilogue or the fused SwiGLU + MXFP4 requant epilogue, and the
// dispatcher that picks its tile shape.
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
//  * Tiles: a workgroup of WGM x WGN waves owns a BM x BN output tile; each
//    wave a (BM/WGM) x (BN/WGN) sub-tile of 32 x 32 accumulators.  K streams
//    in stages of 128 bytes per row (128 e4m3 or 256 e2m1 elements) through a
//    2- or 3-slot LDS ring filled by direct global->LDS loads
//    (global_load_lds_dwordx4: each lane's 16 bytes land at LDS base + 16 *
//    lane, no VGPR staging), issued one or two stages ahead of the matrix
//    cores.  The large FP8 rowwise tile instead streams 64-byte stages
//    through four slots, so two stages stay in flight across each barrier
//    (a 128-byte two-slot ring drains to none at every barrier; measured 1-5 %
//    faster on the prefill shapes), and issues those loads from inline
//    assembly (lds_dma16), so that the only waits before its fragment reads
//    are the ring's own counted ones (4-5 % faster than with the builtin,
//    whose load tracking made the compiler drain the ring every fourth
//    stage).  The 256 x 384 FP8 tile streams 64-byte stages through three
//    slots (four would fill all of LDS), the same way.  The 16-byte chunks
//    of a row are XOR-swizzled (see swz_chunk) so the 16-byte fragment reads of 16
//    consecutive rows hit distinct bank groups; the swizzle is realised by
//    choosing which global chunk each lane fetches.  A stage that runs past
//    the end of K (only the last one, when K bytes are not a multiple of the
//    stage) goes through VGPRs so its tail can be zero-filled.
//  * MX scales: when K is a multiple of 1024 the workgroup stages 32 (or, for
//    the 256 x 256 tile, 16) scale bytes of each of its rows through two LDS
//    buffers with direct loads, one chunk per 32 (16) blocks, and each lane
//    reads its words from there per stage; otherwise each lane loads the 4
//    (e4m3) or 8 (e2m1) scale bytes of its own row for the next stage into
//    registers.  Either way the byte of a lane's block is selected per step.
//  * Ragged groups without host sync: the tile map of gemm_common.h.  Rows
//    past a group's end (columns past N) re-read the last real one and are
//    never stored.
//  * Persistent, XCD-aware schedule: the grid is sized to the resident
//    capacity; workgroup b (dispatched to XCD b % 8) walks logical tiles so
//    that the workgroups resident on one XCD hold consecutive tiles, and the
//    tiles of an expert run in bands of a few M tiles (N outer inside a
//    band), so the tiles on one XCD at a time form a block that shares A and
//    weight panels in that XCD's L2.
#include <cstdlib>
#include <cstring>

#include "gemm_common.h"

namespace mxg {

using namespace gemm;

namespace {

// Prepared weights come in blocks of 256 columns (prepare_weights_kernel).
constexpr int kPrepRows = 256;

// BM x BN output tile, WGM x WGN waves, SLOTS stages of LDS ring (2: one stage
// in flight while one is consumed; 3: two; 4: three), SB K bytes per row per
// stage (128, or 64 for FP8 rowwise: half the LDS per stage, so a 256 x 256
// tile fits four slots and keeps loads in flight across its barriers).
// STREAM_B: the weight
// operand is loaded with the nontemporal cache policy -- for the small
// weight-streaming tile, where each weight panel is read by the few M tiles
// of its expert at about the same time and then never again (measured on
// the decode-shaped workload: 157-164 -> 141-146 us; the large tiles, whose
// weight panels are re-read from L2, were slower with it).
// BPREP: the weights come in the prepared layout (see prepare_weights_kernel).
template <int BM_, int BN_, int WGM_, int WGN_, int SLOTS_ = 3, int MINB_ = 1, bool STREAM_B_ = false, int SB_ = 128,
          bool BPREP_ = false>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, kMinBlocks = MINB_, kSlots = SLOTS_;
    static constexpr int kSB = SB_;
    static constexpr bool kBPrep = BPREP_;
    // direct-to-LDS loads: 16 bytes per lane, kLPR lanes per stage row, so one
    // wave instruction (1 KiB) covers kRPI rows
    static constexpr int kLPR = SB_ / 16, kRPI = 64 / kLPR;
    static constexpr bool kStreamB = STREAM_B_;
    // Fragment buffers per wave: with one wave per SIMD the fragments of step
    // s+1 are read while step s computes (2); with two waves per SIMD the
    // other wave covers the LDS latency and the registers go to accumulators.
    static_assert(SLOTS_ >= 2 && SLOTS_ <= 4, "2- to 4-slot LDS ring");
    static_assert(SB_ == 128 || SB_ == 64, "stage rows of 128 or 64 bytes");
    static constexpr int kWaves = WGM * WGN, kThreads = kWave * kWaves;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int kFragBufs = kWaves >= 8 ? 1 : 2;
    static_assert(TM >= 1 && TN >= 1, "wave tile below one 32x32 accumulator");
    static_assert(BM % (kRPI * kWaves) == 0 && BN % (kRPI * kWaves) == 0, "loader: whole row groups per wave");
};

// One fragment of a 64-deep K step, read from LDS: A row block i (from sa)
// or B column block j (from sb) of this wave's sub-tile.
template <class TL, int FMT>
__device__ __forceinline__ v8i load_frag(const uint8_t* __restrict__ base, int s, int row, int h) {
    if constexpr (Fmt<FMT>::kFP4) {
        const uint4 x = *reinterpret_cast<const uint4*>(base + swz<TL::kSB>(row, 2 * s + h));
        return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    } else {
        const uint4 x0 = *reinterpret_cast<const uint4*>(base + swz<TL::kSB>(row, 4 * s + h));
        const uint4 x1 = *reinterpret_cast<const uint4*>(base + swz<TL::kSB>(row, 4 * s + 2 + h));
        return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
}

// The TM x TN matrix-core ops of row block i at step s.  Scale words arrive
// shifted right by 8h (h = lane half), so block 2s + h of the stage is byte
// 2(s%2) of word s/2 for every lane: a constant byte select.
template <class TL, int FMT, int SEL>
__device__ __forceinline__ void mma_row_sel(int i, int s, const v8i& a, const v8i (&bf)[TL::TN],
                                            const uint32_t (&wa)[TL::TM][Fmt<FMT>::kWords],
                                            const uint32_t (&wb)[TL::TN][Fmt<FMT>::kWords],
                                            v16f (&acc)[TL::TM][TL::TN]) {
    using F = Fmt<FMT>;
#pragma unroll
    for (int j = 0; j < TL::TN; ++j) {
        if constexpr (F::kMX)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bf[j], acc[i][j], F::kTypeCode,
                                                                         F::kTypeCode, SEL, (int)wa[i][s >> 1], SEL,
                                                                         (int)wb[j][s >> 1]);
        else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
}
template <class TL, int FMT>
__device__ __forceinline__ void mma_row(int i, int s, const v8i& a, const v8i (&bf)[TL::TN],
                                        const uint32_t (&wa)[TL::TM][Fmt<FMT>::kWords],
                                        const uint32_t (&wb)[TL::TN][Fmt<FMT>::kWords],
                                        v16f (&acc)[TL::TM][TL::TN]) {
    if (s & 1) mma_row_sel<TL, FMT, 2>(i, s, a, bf, wa, wb, acc);  // s is unrolled: the branch folds
    else mma_row_sel<TL, FMT, 0>(i, s, a, bf, wa, wb, acc);
}

// NVFP4 on the f16 matrix cores.  gfx950's scaled MFMA takes only E8M0
// block scales per 32 elements, so an NVFP4 element (e2m1 code times its
// block's E4M3 scale) is turned into an exact f16 value instead: the scaled
// convert multiplies by the scale's power of two (it uses only the exponent
// of its fp32 scale operand -- measured), a packed f16 multiply by the scale's
// 1.xxx mantissa finishes it; the product has at most 6 significant bits and
// lies in [2^-10, 2688] or is 0, so both steps are exact.  Lane half h holds
// K 32h .. 32h+31 of each 64-deep step (16 bytes, two 16-element blocks, as
// the FP4 fragments are laid out); quarter q of them (8 elements) is the
// lane's operand of the q-th 32x32x16 f16 MFMA, with the same K mapping on
// the B side, so the products pair up.
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void nv_split_scale(uint32_t code, float& pow2, h2v& mant) {
    const float v = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
    const uint32_t b = __float_as_uint(v);
    pow2 = __uint_as_float(b & 0x7f800000u);
    const _Float16 m = (_Float16)__uint_as_float((b & 0x007fffffu) | 0x3f800000u);
    mant = h2v{m, m};
}

__device__ __forceinline__ h8v nv_dequant8(uint32_t codes, float pow2, h2v mant) {
    const h2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 0) * mant;
    const h2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 1) * mant;
    const h2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 2) * mant;
    const h2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, pow2, 3) * mant;
    return h8v{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// All K steps of one NVFP4 stage.  wa / wb: the stage's 16 scale bytes of
// each of this lane's rows / columns, word s = blocks 4s .. 4s+3.
template <class TL>
__device__ __forceinline__ void mma_stage_nv(const uint8_t* __restrict__ sa, const uint8_t* __restrict__ sb, int wm,
                                             int wn, int h, int r32, const uint32_t (&wa)[TL::TM][4],
                                             const uint32_t (&wb)[TL::TN][4], v16f (&acc)[TL::TM][TL::TN]) {
    constexpr int TM = TL::TM, TN = TL::TN;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint4 ra[TM], rb[TN];
        float pa[TM][2], pb[TN][2];
        h2v ma[TM][2], mb[TN][2];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            ra[i] = *reinterpret_cast<const uint4*>(sa + swz<128>(wm * TL::WTM + i * 32 + r32, 2 * s + h));
            const uint32_t w = wa[i][s] >> (16 * h);  // bytes 0, 1: this lane's two blocks
            nv_split_scale(w & 0xffu, pa[i][0], ma[i][0]);
            nv_split_scale((w >> 8) & 0xffu, pa[i][1], ma[i][1]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            rb[j] = *reinterpret_cast<const uint4*>(sb + swz<128>(wn * TL::WTN + j * 32 + r32, 2 * s + h));
            const uint32_t w = wb[j][s] >> (16 * h);
            nv_split_scale(w & 0xffu, pb[j][0], mb[j][0]);
            nv_split_scale((w >> 8) & 0xffu, pb[j][1], mb[j][1]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h8v av[TM], bv[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint32_t c = q == 0 ? ra[i].x : q == 1 ? ra[i].y : q == 2 ? ra[i].z : ra[i].w;
                av[i] = nv_dequant8(c, pa[i][q >> 1], ma[i][q >> 1]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint32_t c = q == 0 ? rb[j].x : q == 1 ? rb[j].y : q == 2 ? rb[j].z : rb[j].w;
                bv[j] = nv_dequant8(c, pb[j][q >> 1], mb[j][q >> 1]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    }
}

// All K steps of one stage.  Two waves per SIMD (one fragment set): the
// other wave covers the LDS latency.  One wave per SIMD: the next step's
// fragments are read while the matrix cores work -- each A fragment is
// replaced right after the ops of its row block, B fragments alternate
// between two sets.
template <class TL, int FMT>
__device__ __forceinline__ void mma_stage(const uint8_t* __restrict__ sa, const uint8_t* __restrict__ sb, int wm,
                                          int wn, int h, int r32,
                                          const uint32_t (&wa_in)[TL::TM][Fmt<FMT>::kWords],
                                          const uint32_t (&wb_in)[TL::TN][Fmt<FMT>::kWords],
                                          v16f (&acc)[TL::TM][TL::TN]) {
    using F = Fmt<FMT>;
    if constexpr (F::kNV) {
        mma_stage_nv<TL>(sa, sb, wm, wn, h, r32, wa_in, wb_in, acc);
        return;
    }
    constexpr int TM = TL::TM, TN = TL::TN, kW = F::kWords;
    constexpr int kSteps = TL::kSB / (F::kFP4 ? 32 : 64);  // 64-deep K steps per stage
    uint32_t wa[TM][kW], wb[TN][kW];
    if constexpr (F::kMX) {
#pragma unroll
        for (int w = 0; w < kW; ++w) {
#pragma unroll
            for (int i = 0; i < TM; ++i) wa[i][w] = wa_in[i][w] >> (8 * h);
#pragma unroll
            for (int j = 0; j < TN; ++j) wb[j][w] = wb_in[j][w] >> (8 * h);
        }
    }
    auto arow = [&](int i) { return wm * TL::WTM + i * 32 + r32; };
    auto brow = [&](int j) { return wn * TL::WTN + j * 32 + r32; };
    if constexpr (kSteps == 1 && TL::kFragBufs == 1 && TN >= 3) {
        // One K step per stage with a wide wave tile (its accumulators leave
        // little room): the B fragments for the whole stage, the A fragments
        // one row block ahead of the matrix cores.  The lane's row offsets are
        // recomputed here from an opaque copy of its row index, so that no
        // per-slot read address is held through the K loop.
        uint32_t rl = (uint32_t)r32;
        __asm__ volatile("" : "+v"(rl));
        const int ra = wm * TL::WTM + (int)rl, rbw = wn * TL::WTN + (int)rl;
        v8i bq[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) bq[j] = load_frag<TL, FMT>(sb, 0, rbw + j * 32, h);
        v8i a_cur = load_frag<TL, FMT>(sa, 0, ra, h);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            v8i a_nxt;
            if (i + 1 < TM) a_nxt = load_frag<TL, FMT>(sa, 0, ra + (i + 1) * 32, h);
            mma_row<TL, FMT>(i, 0, a_cur, bq, wa, wb, acc);
            if (i + 1 < TM) a_cur = a_nxt;
        }
        return;
    }
    v8i af[TM], bf[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = load_frag<TL, FMT>(sa, 0, arow(i), h);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[0][j] = load_frag<TL, FMT>(sb, 0, brow(j), h);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int c = s & 1, n = c ^ 1;
        if constexpr (TL::kFragBufs == 1) {
#pragma unroll
            for (int i = 0; i < TM; ++i) mma_row<TL, FMT>(i, s, af[i], bf[c], wa, wb, acc);
            if (s + 1 < kSteps) {
#pragma unroll
                for (int i = 0; i < TM; ++i) af[i] = load_frag<TL, FMT>(sa, s + 1, arow(i), h);
#pragma unroll
                for (int j = 0; j < TN; ++j) bf[n][j] = load_frag<TL, FMT>(sb, s + 1, brow(j), h);
            }
        } else {
            constexpr int kBPerRow = (TN + TM - 1) / TM;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                mma_row<TL, FMT>(i, s, af[i], bf[c], wa, wb, acc);
                if (s + 1 < kSteps) {
                    af[i] = load_frag<TL, FMT>(sa, s + 1, arow(i), h);
#pragma unroll
                    for (int k = 0; k < kBPerRow; ++k)
                        if (i * kBPerRow + k < TN)
                            bf[n][i * kBPerRow + k] = load_frag<TL, FMT>(sb, s + 1, brow(i * kBPerRow + k), h);
                }
            }
            if (s + 1 < kSteps) {
                // interleave: one matrix-core op, then a share of the next step's LDS reads
                constexpr int kMfma = TM * TN;
                constexpr int kReads = (TM + TN) * (F::kFP4 ? 1 : 2);
#pragma unroll
                for (int q = 0; q < kMfma; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                            // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, (kReads + kMfma - 1) / kMfma, 0);  // DS read
                }
            }
        }
    }
}

// KA: K bytes are a whole number of stages (no partial last stage) and, for
// the MX formats, K is a multiple of 1024 (scale rows a whole number of
// 32-byte chunks), so the scales are staged through LDS (see below) instead
// of loaded per lane.
template <class TL, int FMT, bool SWIGLU, bool KA>
__global__ __launch_bounds__(TL::kThreads, TL::kMinBlocks) void grouped_gemm_kernel(const GemmArgs args) {
    using F = Fmt<FMT>;
    constexpr int BM = TL::BM, BN = TL::BN, NW = TL::kWaves, NT = TL::kThreads;
    constexpr int WTM = TL::WTM, WTN = TL::WTN, TM = TL::TM, TN = TL::TN;
    constexpr int SB = TL::kSB, kLPR = TL::kLPR, kRPI = TL::kRPI;
    static_assert(SB == kStageBytes || (!F::kMX && KA), "64-byte stages: FP8 rowwise with whole stages only");
    constexpr int kAStage = BM * SB, kBStage = BN * SB;
    constexpr int kStage = kAStage + kBStage;
    constexpr int A_J = BM / kRPI / NW, B_J = BN / kRPI / NW;  // 1 KiB load instructions per wave per stage
    constexpr int kWords = F::kWords;                    // scale words per row per stage
    // cache policy of the weight loads (a named constant: written as a
    // conditional expression inside the builtin call, hipcc dropped the
    // kernels' host launch stubs without an error)
    constexpr int kBPolicy = TL::kStreamB ? kCpolNT : 0;
    // MX scales through LDS: every kSclStages stages the workgroup loads the
    // next 32 scale bytes (32 blocks) of each of its BM + BN rows with direct
    // loads (an instruction covers 32 rows, two lanes per row), into one of
    // two buffers; lanes then read their words from LDS.  One request per
    // row per 32 blocks instead of a 4-byte load per row, stage and wave.
    constexpr bool kLdsScales = F::kMX && KA;
    constexpr int kSclRows = BM + BN;
    // 32-byte chunks where both buffers fit beside the ring, else 16
    constexpr int kSclBytes = TL::kSlots * kStage + 2 * kSclRows * 32 + 8192 <= 160 * 1024 ? 32 : 16;
    constexpr int kSclStages = kSclBytes / F::kBlocks;
    static_assert(!kLdsScales || (TL::kSlots == 2 && BM % 32 == 0 && BN % 32 == 0),
                  "LDS scales: two ring slots, whole 32-row groups");

    // Ring slots as distinct objects: the compiler can then tell the
    // direct-to-LDS loads into one slot from the fragment reads of another and
    // does not serialise them.  kSlots - 1 stages are in flight while one is
    // consumed.
    constexpr int kSlots = TL::kSlots;
    __shared__ __attribute__((aligned(16))) uint8_t s_ring0[kStage];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring1[kStage];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring2[kSlots > 2 ? kStage : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring3[kSlots > 3 ? kStage : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_scl0[kLdsScales ? kSclRows * kSclBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t s_scl1[kLdsScales ? kSclRows * kSclBytes : 16];
    __shared__ uint32_t s_pre[kMaxGroups + 1];
    __shared__ uint32_t s_wave[NW];
    // The tile's per-row epilogue factor -- FP8 rowwise: a_scale of the row;
    // NVFP4: the expert scale times, fused with a row scale, the row's scale
    // -- loaded at the start of the tile (the loads land behind the K loop) so
    // that the epilogue reads it from LDS instead of issuing global loads
    // after the K loop.
    constexpr bool kRowFactor = !F::kMX || F::kNV;
    __shared__ float s_rowf[kRowFactor ? BM : 1];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / TL::WGN, wn = wave % TL::WGN;
    const int h = lane >> 5, r32 = lane & 31;
    const int G = args.G;

    build_tile_prefix<NT, BM>(args, s_pre, s_wave);
    const int64_t total_tiles = (int64_t)s_pre[G] * args.ntiles_n;
    const int64_t row_bytes = args.row_bytes;
    const int nkt = (int)((row_bytes + SB - 1) / SB);
    const bool k_tail = !KA && (row_bytes % SB) != 0;  // the last stage is partial
    const int64_t nblk = args.K / F::kBlockElems;  // scale bytes per row

    const WorkSplit ws = work_split(total_tiles, gridDim.x);
    for (int64_t W = xcd_remap(blockIdx.x, gridDim.x); W < ws.items; W += gridDim.x) {
        const TileCoord tc = uniform_coord(locate_item<BM, BN>(args, s_pre, ws, W));
        if (tc.cols_in <= 0) continue;  // the empty second half of a last, narrow tile (uniform)
        const int e = tc.e;
        const int64_t m0 = tc.m0, n0 = tc.n0, n_end = tc.n_end;
        int64_t m_end = tc.m_end;  // one past the last row stored (a padded scale layout can lower it)
        const int rows_in = tc.rows_in, cols_in = tc.cols_in;
        // A wave whose sub-tile lies wholly past the group's last row or past
        // the last column (partial M tiles, half tiles of a split round)
        // skips its matrix-core work; the loads stay shared.
        const bool wave_live = wm * WTM < rows_in && wn * WTN < cols_in;  // wave-uniform
        // (rows past the group's end take the last real row's factor; never stored)
        if constexpr (!F::kMX) {
            const float* as = static_cast<const float*>(args.as);
            for (int i = tid; i < BM; i += NT) s_rowf[i] = as[m0 + (i < rows_in ? i : rows_in - 1)];
        } else if constexpr (F::kNV) {
            const float es_e = args.es[e];
            for (int i = tid; i < BM; i += NT)
                s_rowf[i] = SWIGLU && args.rs ? es_e * bf16_to_f32(args.rs[m0 + (i < rows_in ? i : rows_in - 1)])
                                              : es_e;
        }

        // ---- operand sources: tile base (uniform) + 32-bit per-lane offsets;
        // load j of a wave covers rows r0 + kRPI NW j .. + kRPI - 1, kLPR
        // chunks each (1 KiB of the slot).  Rows past the group / columns past N re-read the last
        // real one.  With an even wave count the swizzled chunk of a lane is
        // the same for every j (the swizzle reads row bits the step
        // kRPI NW j leaves alone).  The offsets are held in registers (one per
        // load) through the K loop, except in the eight-wave MX kernel, which
        // runs out of registers (spills in the K loop stall it on the
        // prefetch): there they are recomputed per stage from two registers.
        static_assert(NW % 2 == 0, "per-lane chunk independent of the load index");
        constexpr bool kLeanOffsets = F::kMX && NW >= 8;
        const uint8_t* a_base = args.a + m0 * row_bytes;
        // Prepared weights: stage kt of 256-column block nb is the 256 x
        // 64-byte image at ((e * ceil(N / 256) + nb) * nkt + kt) * 16 KiB; the
        // tile starts at row n0 % 256 of block n0 / 256 and a 384-column tile
        // runs into the next block.  One load instruction reads 1 KiB.
        static_assert(!TL::kBPrep || (!F::kMX && SB == 64), "prepared weights: FP8 64-byte-stage ring");
        const int64_t prep_ntn = (args.N + kPrepRows - 1) / kPrepRows;
        const uint8_t* b_base = TL::kBPrep
                                    ? args.b + ((int64_t)e * prep_ntn + n0 / kPrepRows) * nkt * (int64_t)(kPrepRows * SB)
                                    : args.b + ((int64_t)e * args.N + n0) * row_bytes;
        const int r0 = wave * kRPI + lane / kLPR;
        const uint32_t chunk16 = (uint32_t)swz_chunk<SB>(r0, lane % kLPR) << 4;
        const uint32_t rb32 = (uint32_t)row_bytes;
        auto op_off = [&](int rbase, int j, int live) {
            const int r = rbase + kRPI * NW * j;
            return (uint32_t)(r < live ? r : live - 1) * rb32 + chunk16;
        };
        uint32_t a_off[A_J], b_off[B_J];
        if constexpr (!kLeanOffsets) {
#pragma unroll
            for (int j = 0; j < A_J; ++j) a_off[j] = op_off(r0, j, rows_in);
#pragma unroll
            for (int j = 0; j < B_J; ++j) b_off[j] = op_off(r0, j, cols_in);
        }
        // Offsets (or, lean, the row base) pass through an empty asm
        // statement in each stage, so the compiler does not hoist 64-bit
        // per-lane addresses out of the K loop (nor, lean, keep every offset
        // live through it); addresses stay a uniform base plus a 32-bit
        // offset.
        auto opaque = [](uint32_t v) {
            __asm__ volatile("" : "+v"(v));
            return v;
        };
        // The rings of 64-byte stages issue their direct loads from inline
        // assembly (see lds_dma16): their K loops issue no other vector-memory
        // instruction (FP8 rowwise: no scale loads; no register spills).
        constexpr bool kAsmDma = SB == 64;
        static_assert(!kAsmDma || !F::kMX, "assembly ring loads: FP8 rowwise only");
        auto issue_stage = [&](int kt, uint8_t* slot) {
            const uint8_t* ak = a_base + (int64_t)kt * SB;
            const uint8_t* bk = b_base + (int64_t)kt * (TL::kBPrep ? kPrepRows * SB : SB);
            const int rb = kLeanOffsets ? (int)opaque((uint32_t)r0) : r0;
#pragma unroll
            for (int j = 0; j < A_J; ++j) {
                const uint32_t off = kLeanOffsets ? op_off(rb, j, rows_in) : opaque(a_off[j]);
                if constexpr (kAsmDma)
                    lds_dma16<false>(ak, off, lds_addr(slot + (wave + NW * j) * 1024));
                else
                    __builtin_amdgcn_global_load_lds((gptr_t)(ak + off), (lptr_t)(slot + (wave + NW * j) * 1024), 16,
                                                     0, 0);
            }
#pragma unroll
            for (int j = 0; j < B_J; ++j) {
                uint32_t off = kLeanOffsets ? op_off(rb, j, cols_in) : opaque(b_off[j]);
                if constexpr (TL::kBPrep) {
                    // Load groups wholly past the tile's columns re-read its
                    // last real group; a group lies in one 256-column block
                    // (n0 and kRPI are multiples of 16).  The lane term passes
                    // through the empty asm, the rest is uniform; unsigned, as
                    // two blocks of K * 256 bytes reach 2^31 at K = MXG_MAX_K.
                    const int q = wave + NW * j;
                    const int c = (int)(n0 % kPrepRows) + (q * kRPI < cols_in ? q : (cols_in - 1) / kRPI) * kRPI;
                    off = opaque((uint32_t)lane * 16u) + (uint32_t)(c / kPrepRows) * (uint32_t)nkt * (uint32_t)(kPrepRows * SB) +
                          (uint32_t)((c % kPrepRows) * SB);
                }
                if constexpr (kAsmDma)
                    lds_dma16<TL::kStreamB>(bk, off, lds_addr(slot + kAStage + (wave + NW * j) * 1024));
                else
                    __builtin_amdgcn_global_load_lds((gptr_t)(bk + off),
                                                     (lptr_t)(slot + kAStage + (wave + NW * j) * 1024), 16, 0,
                                                     kBPolicy);
            }
        };
        // The partial last stage: VGPR loads with the K tail zero-filled.
        uint4 ta[A_J], tb[B_J];
        auto load_tail = [&](int kt) {
            const int64_t kb = (int64_t)kt * SB;
            const int c_lo = lane % kLPR;  // physical chunk; the logical one depends on the row
#pragma unroll
            for (int j = 0; j < A_J; ++j) {
                const int r = (wave + NW * j) * kRPI + lane / kLPR;
                const bool in = kb + swz_chunk<SB>(r, c_lo) * 16 < row_bytes;
                ta[j] = in ? *reinterpret_cast<const uint4*>(a_base + kb + op_off(r0, j, rows_in)) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < B_J; ++j) {
                const int r = (wave + NW * j) * kRPI + lane / kLPR;
                const bool in = kb + swz_chunk<SB>(r, c_lo) * 16 < row_bytes;
                tb[j] = in ? *reinterpret_cast<const uint4*>(b_base + kb + op_off(r0, j, cols_in)) : make_uint4(0, 0, 0, 0);
            }
        };
        auto store_tail = [&](uint8_t* slot) {
#pragma unroll
            for (int j = 0; j < A_J; ++j) *reinterpret_cast<uint4*>(slot + (wave + NW * j) * 1024 + lane * 16) = ta[j];
#pragma unroll
            for (int j = 0; j < B_J; ++j)
                *reinterpret_cast<uint4*>(slot + kAStage + (wave + NW * j) * 1024 + lane * 16) = tb[j];
        };

        // ---- MX scale words of this lane's rows / columns, one stage ahead.
        // A padded A-scale layout moves the tile's first scale row (a tile
        // never spans groups).  Rows whose scale row lies at or past the end
        // of the scale tensor are not stored (their outputs are left
        // untouched); their scale reads are clamped to the last row that
        // exists, as rows past a group's end are.
        int64_t sa_row0 = m0;
        int rows_sc = rows_in;  // rows of the tile whose scale rows exist
        if (F::kMX && args.asoff) {
            sa_row0 = (int64_t)args.asoff[tc.g] + (m0 - tc.glo);
            const int64_t avail = args.as_rows - sa_row0;
            if (avail <= 0) continue;  // uniform; nothing to store
            if (avail < rows_in) {
                rows_sc = (int)avail;
                m_end = m0 + avail;
            }
        }
        const uint8_t* sa_base = static_cast<const uint8_t*>(args.as) + sa_row0 * nblk;
        const uint8_t* sb_base = static_cast<const uint8_t*>(args.bs) + ((int64_t)e * args.N + n0) * nblk;
        uint32_t sa_off[TM], sb_off[TN];
        uint32_t wa[TM][kWords], wb[TN][kWords];
        if constexpr (F::kMX) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + r32;
                sa_off[i] = (uint32_t)((r < rows_sc ? r : rows_sc - 1) * nblk);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + r32;
                sb_off[j] = (uint32_t)((r < cols_in ? r : cols_in - 1) * nblk);
            }
        }
        // LDS-staged scales: chunk c (32 bytes per row from block 32c) into
        // buffer `buf`, rows 0 .. BM-1 of A then BM .. BM+BN-1 of B, row r at
        // byte 32r; 32-row group q is loaded by wave q % NW (lane l: row
        // 32q + l/2).  With 32-byte chunks the two 16-byte halves of a row
        // trade places when bit 3 of the row is set (lane l fetches half
        // (l % 2) ^ ((l >> 4) & 1)): the 32 rows a 4-byte scale read covers
        // then fall on 16 bank groups instead of 8 (two-way instead of
        // four-way LDS bank conflicts, the least a 4-byte read of one word
        // per row allows).
        constexpr int kSclRowsPerLoad = 1024 / kSclBytes;
        constexpr int kSclGroups = kSclRows / kSclRowsPerLoad;
        constexpr int kSclPerWave = (kSclGroups + NW - 1) / NW;
        static_assert(!kLdsScales || (WTM % 32 == 0 && WTN % 32 == 0),
                      "LDS scales: wave row blocks start on 32-row boundaries");
        const uint8_t* scl_base[kSclPerWave];
        uint32_t scl_off[kSclPerWave];
        if constexpr (kLdsScales) {
#pragma unroll
            for (int k = 0; k < kSclPerWave; ++k) {
                const int q = wave + NW * k;
                const int r = q * kSclRowsPerLoad + lane / (kSclBytes / 16);
                const bool in_a = q * kSclRowsPerLoad < BM;  // wave-uniform
                const int half = kSclBytes == 32 ? (lane % 2) ^ ((lane >> 4) & 1) : 0;
                scl_base[k] = in_a ? sa_base : sb_base;
                scl_off[k] = (in_a ? (uint32_t)((r < rows_sc ? r : rows_sc - 1) * nblk)
                                   : (uint32_t)((r - BM < cols_in ? r - BM : cols_in - 1) * nblk)) +
                             16 * half;
            }
        }
        auto issue_scales = [&](int c, uint8_t* buf) {
#pragma unroll
            for (int k = 0; k < kSclPerWave; ++k)
                if (wave + NW * k < kSclGroups)  // wave-uniform
                    __builtin_amdgcn_global_load_lds((gptr_t)(scl_base[k] + kSclBytes * c + opaque(scl_off[k])),
                                                     (lptr_t)(buf + (wave + NW * k) * 1024), 16, 0, 0);
        };
        // this lane's scale words for position `pos` (stage within a chunk);
        // the row's bit 3 is r32's (row blocks start on 32-row boundaries), so
        // byte b of the chunk sits at b + sx in the first half, b - sx in the
        // second
        const int sx = kLdsScales && kSclBytes == 32 ? ((r32 >> 3) & 1) * 16 : 0;
        auto read_scales = [&](const uint8_t* buf, int pos, uint32_t (&xa)[TM][kWords], uint32_t (&xb)[TN][kWords]) {
#pragma unroll
            for (int w = 0; w < kWords; ++w) {
                const int b = (pos * kWords + w) * 4;
                const int bs = b < 16 ? b + sx : b - sx;
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    xa[i][w] = *reinterpret_cast<const uint32_t*>(buf + (wm * WTM + i * 32 + r32) * kSclBytes + bs);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    xb[j][w] = *reinterpret_cast<const uint32_t*>(buf + (BM + wn * WTN + j * 32 + r32) * kSclBytes +
                                                                  bs);
            }
        };
        auto load_scales = [&](int kt, uint32_t (&xa)[TM][kWords], uint32_t (&xb)[TN][kWords]) {
            const int64_t b0 = (int64_t)kt * F::kBlocks;
#pragma unroll
            for (int w = 0; w < kWords; ++w) {
#pragma unroll
                for (int i = 0; i < TM; ++i) xa[i][w] = scale_word(sa_base + b0 + 4 * w + sa_off[i], nblk - b0 - 4 * w);
#pragma unroll
                for (int j = 0; j < TN; ++j) xb[j][w] = scale_word(sb_base + b0 + 4 * w + sb_off[j], nblk - b0 - 4 * w);
            }
        };

        v16f acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};

        // ---- prologue: stages 0 .. kSlots-2 into the first slots
        auto put_stage = [&](int kt, uint8_t* slot) {
            if (k_tail && kt == nkt - 1) {
                load_tail(kt);
                store_tail(slot);
            } else {
                issue_stage(kt, slot);
            }
        };
        constexpr int L = A_J + B_J;  // direct loads per wave per stage
        // wait until this wave's loads of the stage needed next have landed,
        // leaving those of the `later` stages issued after it in flight (the
        // loads land in issue order), then the workgroup barrier
        auto barrier_leaving = [&](int later) {
            if (later >= 2) stage_barrier<2 * L>();
            else if (later == 1) stage_barrier<L>();
            else stage_barrier<0>();
        };
        if constexpr (kSlots == 4) {
            static_assert(KA, "four slots: whole stages only");
            // The previous tile's output stores share the vector-memory counter
            // with these loads and may complete out of order with them; let
            // them finish first so the counted waits see only this tile's stages.
            wait_vmem<0>();
            issue_stage(0, s_ring0);
            if (nkt > 1) issue_stage(1, s_ring1);
            if (nkt > 2) issue_stage(2, s_ring2);
            barrier_leaving(nkt - 1 < 2 ? nkt - 1 : 2);
        } else {
            put_stage(0, s_ring0);
            if (kSlots > 2 && nkt > 1) put_stage(1, s_ring1);
            if constexpr (kLdsScales) issue_scales(0, s_scl0);
            else if constexpr (F::kMX) load_scales(0, wa, wb);
            wait_vmem<0>();
            __syncthreads();
        }

        // One stage: the matrix cores consume `cur` (stage kt) while stage
        // kt + kSlots - 1 streams into `pf` (and, with three slots, stage kt+1,
        // issued one stage earlier, lands); the slots rotate, so the loop is
        // unrolled by kSlots.
        constexpr int D = kSlots - 1;  // prefetch distance in stages
        auto stage = [&](int kt, const uint8_t* cur, uint8_t* pf) {
            const bool pf_on = kt + D < nkt;
            const bool pf_tail = pf_on && k_tail && kt + D == nkt - 1;
            uint32_t na[TM][kWords], nb[TN][kWords];
            if constexpr (F::kMX)
                if (kt + 1 < nkt) load_scales(kt + 1, na, nb);
            if (pf_on) {
                if (pf_tail) load_tail(kt + D);
                else issue_stage(kt + D, pf);
            }
            if (wave_live) mma_stage<TL, FMT>(cur, cur + kAStage, wm, wn, h, r32, wa, wb, acc);
            if (pf_tail) store_tail(pf);
            if constexpr (F::kMX)
                if (kt + 1 < nkt) {
#pragma unroll
                    for (int w = 0; w < kWords; ++w) {
#pragma unroll
                        for (int i = 0; i < TM; ++i) wa[i][w] = na[i][w];
#pragma unroll
                        for (int j = 0; j < TN; ++j) wb[j][w] = nb[j][w];
                    }
                }
            // stage kt+1 (and its scales) must have landed; with three slots
            // stage kt+2's direct loads, the most recent ones, may stay in
            // flight, with four slots those of kt+2 and kt+3
            if constexpr (D == 3) {
                const int later = nkt - 2 - kt;
                barrier_leaving(later < 2 ? (later > 0 ? later : 0) : 2);
            } else if (D == 2 && pf_on && !pf_tail) {
                stage_barrier<L>();
            } else {
                stage_barrier<0>();
            }
        };
        // With LDS scales: the stage also reads its scale words from `scur`
        // (position pos of the chunk) and, in a chunk's last stage, starts the
        // next chunk into `snext`, which the chunk before last used.  Slots
        // and scale buffers rotate, so that loop is unrolled by
        // 2 * kSclStages.
        auto stage_lds = [&](int kt, const uint8_t* cur, uint8_t* pf, const uint8_t* scur, uint8_t* snext,
                             int pos) {
            const bool pf_on = kt + 1 < nkt;
            uint32_t xa[TM][kWords], xb[TN][kWords];
            if (wave_live) read_scales(scur, pos, xa, xb);
            if (pf_on) issue_stage(kt + 1, pf);
            if (pos == kSclStages - 1 && pf_on) issue_scales((kt + 1) / kSclStages, snext);
            if (wave_live) mma_stage<TL, FMT>(cur, cur + kAStage, wm, wn, h, r32, xa, xb, acc);
            stage_barrier<0>();
        };
        if constexpr (kLdsScales) {
            constexpr int U = 2 * kSclStages;
            for (int kt = 0; kt < nkt; kt += U) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (kt + u < nkt)
                        stage_lds(kt + u, u % 2 ? s_ring1 : s_ring0, u % 2 ? s_ring0 : s_ring1,
                                  (u / kSclStages) % 2 ? s_scl1 : s_scl0, (u / kSclStages) % 2 ? s_scl0 : s_scl1,
                                  u % kSclStages);
            }
        } else if constexpr (kSlots == 4) {
            for (int kt = 0; kt < nkt; kt += 4) {
                stage(kt, s_ring0, s_ring3);
                if (kt + 1 < nkt) stage(kt + 1, s_ring1, s_ring0);
                if (kt + 2 < nkt) stage(kt + 2, s_ring2, s_ring1);
                if (kt + 3 < nkt) stage(kt + 3, s_ring3, s_ring2);
            }
        } else if constexpr (kSlots == 3) {
            for (int kt = 0; kt < nkt; kt += 3) {
                stage(kt, s_ring0, s_ring2);
                if (kt + 1 < nkt) stage(kt + 1, s_ring1, s_ring0);
                if (kt + 2 < nkt) stage(kt + 2, s_ring2, s_ring1);
            }
        } else {
            for (int kt = 0; kt < nkt; kt += 2) {
                stage(kt, s_ring0, s_ring1);
                if (kt + 1 < nkt) stage(kt + 1, s_ring1, s_ring0);
            }
        }

        // ---- epilogue.  The output tile is staged in LDS as bf16 rows (the
        // ring is free: the last stage ended at a barrier), spread over the
        // slots, then written out in coalesced 16-byte pieces -- or, fused,
        // requantized from there.
        constexpr int kRowsPerSlot = kStage / (BN * 2);
        // one staging pass when the whole tile fits the ring, else two (half
        // of every wave's row blocks each)
        constexpr int kPasses = kSlots * kRowsPerSlot >= BM ? 1 : 2;
        static_assert(kSlots * kRowsPerSlot >= BM / kPasses, "staging pass must fit the LDS ring");
        static_assert(!SWIGLU || kPasses == 1, "fused epilogue: whole tile staged");
        auto srow = [&](int row) -> uint16_t* {
            uint8_t* base = row < kRowsPerSlot ? s_ring0 : row < 2 * kRowsPerSlot ? s_ring1
                          : row < 3 * kRowsPerSlot ? s_ring2 : s_ring3;
            return reinterpret_cast<uint16_t*>(base + (row % kRowsPerSlot) * BN * 2);
        };
        if constexpr (!SWIGLU) {
            // The two-pass tile takes the lane indices through the empty asm
            // here, so that its staging addresses are computed per tile, not
            // hoisted out of the tile loop and held through the K loop.
            const int eh = kPasses > 1 ? (int)opaque((uint32_t)h) : h;
            const int e32 = kPasses > 1 ? (int)opaque((uint32_t)r32) : r32;
            // out = bf16((acc * a_scale[row]) * b_scale[col]) for FP8 rowwise,
            // bf16(acc * expert_scale[e]) for NVFP4
            auto value = [&](int i, int j, int r, float sbv) {
                float v = acc[i][j][r];
                if constexpr (kRowFactor) v = v * s_rowf[wm * WTM + i * 32 + 8 * (r >> 2) + 4 * eh + (r & 3)];
                if constexpr (!F::kMX) v = v * sbv;
                return (uint16_t)f32_to_bf16(v);
            };
            auto b_scale = [&](int j) {
                const int64_t col = n0 + wn * WTN + j * 32 + e32;
                float sbv = 1.0f;
                if constexpr (!F::kMX)
                    if (col < n_end) sbv = static_cast<const float*>(args.bs)[(int64_t)e * args.N + col];
                return sbv;
            };
            // rows of c start on 16 bytes (a two-pass tile is launched only
            // then: its accumulators leave no room for per-element stores)
            if (kPasses > 1 || (args.N & 7) == 0) {
                // Pass p stages row blocks [p TM/kPasses, (p+1) TM/kPasses) of
                // every wave (one pass: all of them); staged row s is tile row
                // (s / kHalf) WTM + p kHalf + s % kHalf (one pass: s).  The
                // accumulators of a pass die as it is staged.
                constexpr int kIPer = TM / kPasses, kHalf = WTM / kPasses;
                constexpr int kPassRows = BM / kPasses;
                static_assert(TM % kPasses == 0, "whole row blocks per pass");
#pragma unroll
                for (int pass = 0; pass < kPasses; ++pass) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        if (i / kIPer != pass) continue;  // folds: i and pass are unrolled
#pragma unroll
                        for (int j = 0; j < TN; ++j) {
                            const float sbv = b_scale(j);
                            const int col = wn * WTN + j * 32 + e32;
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                srow(wm * kHalf + (i - pass * kIPer) * 32 + 8 * (r >> 2) + 4 * eh + (r & 3))[col] =
                                    value(i, j, r, sbv);
                        }
                    }
                    __syncthreads();
                    constexpr int kPieces = BN / 8;  // 16-byte pieces per tile row
#pragma unroll 1
                    for (int q = tid; q < kPassRows * kPieces; q += NT) {
                        const int s = q / kPieces, pc = q % kPieces;
                        const int row = kPasses == 1 ? s : (s / kHalf) * WTM + pass * kHalf + s % kHalf;
                        const int64_t grow = m0 + row, gcol = n0 + pc * 8;
                        if (grow < m_end && gcol < n_end)
                            store_stream16(args.c + grow * args.N + gcol,
                                           *reinterpret_cast<const uint4*>(srow(s) + pc * 8));
                    }
                    if (pass + 1 < kPasses) __syncthreads();  // the next pass reuses the staging rows
                }
            } else if constexpr (kPasses == 1) {
#pragma unroll
                for (int i = 0; i < TM; ++i) {
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int64_t col = n0 + wn * WTN + j * 32 + r32;
                        const float sbv = b_scale(j);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                            if (row < m_end && col < n_end) args.c[row * args.N + col] = value(i, j, r, sbv);
                        }
                    }
                }
            }
        } else {
            // Requant rows of 32 outputs with the same code the standalone
            // activation kernel runs.
            // (NVFP4: gate/up = bf16(acc * fl32(expert_scale * row_scale)),
            // requant to NVFP4 blocks of 16 under y's tensor scale.)
            static_assert(BN % 64 == 0, "fused tile must hold whole 32-output blocks");
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = wn * WTN + j * 32 + r32;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        float v = acc[i][j][r];
                        if constexpr (F::kNV) v = v * s_rowf[row];
                        srow(row)[col] = (uint16_t)f32_to_bf16(v);
                    }
                }
            }
            __syncthreads();
            constexpr int kBlk = BN / 64;  // 32-output blocks per tile row
            constexpr int kUnits = BM * kBlk;
            const int l4 = tid & 3;
            const int64_t I = args.N / 2;
            // units cover whole 4-lane groups, so every lane runs the shuffles
#pragma unroll 1
            for (int u = tid >> 2; u < kUnits; u += NT / 4) {
                const int row = u / kBlk, blk = u % kBlk;
                const uint4* src = reinterpret_cast<const uint4*>(srow(row) + blk * 64 + l4 * 16);
                float gu[16];
                unpack8(src[0], gu);
                unpack8(src[1], gu + 8);
                float y[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = bf16_to_f32(f32_to_bf16(silu_mul(gu[2 * k], gu[2 * k + 1])));
                const int64_t grow = m0 + row;
                const int64_t gblk = n0 / 64 + blk;
                const bool store = grow < m_end && n0 + blk * 64 < n_end;
                if constexpr (F::kNV) {
                    // lanes (0, 1) and (2, 3) of the group each form a 16-output block
                    uint32_t sc;
                    const uint32_t code = nv_encode8(y, args.ysf[e], sc);
                    const int64_t unit = gblk * 4 + l4;  // 8-output unit within the row
                    if (store) {
                        *reinterpret_cast<uint32_t*>(args.yq + grow * (I / 2) + unit * 4) = code;
                        if ((l4 & 1) == 0) args.ys[grow * (I / 16) + (unit >> 1)] = (uint8_t)sc;
                    }
                } else {
                    uint2 code;
                    const int X = mx_encode8<true>(y, code);
                    if (store)
                        mx_store8<true>(code, X, args.yq + grow * (I / 2), args.ys + grow * (I / 32), gblk * 4 + l4,
                                        l4);
                }
            }
        }
        __syncthreads();  // LDS is reused by the next tile's prologue
    }
}

template <class TL, int FMT, bool SWIGLU, bool KA>
hipError_t launch_tile(const GemmProblem& p, hipStream_t stream, int mband) {
    auto kernel = grouped_gemm_kernel<TL, FMT, SWIGLU, KA>;
    static thread_local int occ_device = -1, occ = 0;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (occ_device != dev) {
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, TL::kThreads, 0);
        if (err != hipSuccess) return err;
        occ_device = dev;
    }
    int64_t grid = 0;
    const GemmArgs a = make_args(p, TL::BM, TL::BN, mband, occ, &grid);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(TL::kThreads), 0, stream, a);
    return hipGetLastError();
}

// Tile shapes and tile orders, chosen by measurement on MI355X (ragged
// workloads of the benchmark): FP8 rowwise with many rows per group (and
// prepared weights always) -> 256-row tiles with eight waves in bands of 4 M
// tiles: 256 x 384 in three 64-byte-stage slots (a sixth fewer operand bytes
// per FLOP than 256 x 256; its 192 accumulators per lane fit beside the K
// loop only with the loop's offsets and fragment addresses recomputed per
// stage and the epilogue staged in two passes; prefill shape 504.6 -> 465.5
// us, bit-identical) where wide_fp8_pays says so, else 256 x 256 (64-byte
// stages in four slots when K is a multiple of 64, else 128-byte stages in
// two); MX formats with K a multiple of
// 1024 (LDS-staged scales) -> with at least 384 rows per group on average
// the eight-wave 256 x 256 tile with 16-byte scale chunks, else the
// eight-wave 192 x 256 tile in bands of 8 M tiles (at 170-270 rows per group
// it streams ~13 % fewer operand rows than 128 x 256 and pads far less than
// 256 x 256: MXFP8 and fused MXFP4 8-17 % faster than 128 x 256; at 512 rows
// per group 256 x 256 stays 3-4 % ahead); other MX shapes -> 128 x 256 with
// four waves and three slots; few rows per group (decode-like, weight
// streaming) -> 32-row tiles, many of them, walked N-outer so the M tiles of
// an expert share each weight panel in L2: FP8 rowwise 32 x 256 with two
// slots (decode workload 140 -> 136 us against 32 x 128 with three; 32 x 512,
// three slots, or 32 x 64 / 32 x 128 with two were slower), MX 32 x 128 with
// three slots.
using TileLargeFp8 = Tile<256, 256, 2, 4, 4, 1, false, 64>;   // whole 64-byte stages
using TileLargeFp8Prep = Tile<256, 256, 2, 4, 4, 1, false, 64, true>;  // the same, prepared weights
using TileWideFp8Prep = Tile<256, 384, 2, 4, 3, 1, false, 64, true>;   // 384 columns, prepared weights (120 KiB ring)
using TileWideFp8 = Tile<256, 384, 2, 4, 3, 1, false, 64>;              // the same on row-major weights
using TileLargeFp8Tail = Tile<256, 256, 2, 4, 2>;              // K bytes not a multiple of 128
using TileLargeMx = Tile<128, 256, 2, 2, 3>;
using TileLargeMxKA = Tile<128, 256, 2, 2, 2>;
using TileLargeMxKA8 = Tile<256, 256, 2, 4, 2>;
using TileMx192 = Tile<192, 256, 2, 4, 2>;
using TileSmall = Tile<32, 128, 1, 4, 3, 1, true>;
using TileSmallFp8 = Tile<32, 256, 1, 4, 2, 1, true>;
constexpr int kBandLarge = 4, kBandMx = 8, kBandNOuter = 1 << 30;
constexpr int64_t kTallRows = 384;

// Prepared weights (FP8 rowwise, K a multiple of 64): element (e, n, k) of the
// [E, N, K] codes goes to tile nt = n / 256, stage kt = k / 64, row r = n % 256
// of a 256 x 64-byte block (the block the 256 x 256 ring copies to LDS as
// it is; the 256 x 384 ring copies one and a half of them), at byte r * 64 +
// 16 * swz_chunk<64>(r, (k % 64) / 16) + k % 16, the blocks ordered (e, nt,
// kt); rows past N are zero.  One 16-byte piece per
// thread.
__global__ __launch_bounds__(256) void prepare_weights_kernel(const uint8_t* __restrict__ b, int64_t E, int64_t N,
                                                              int64_t K, uint8_t* __restrict__ out) {
    constexpr int BN = kPrepRows, SB = TileLargeFp8Prep::kSB;
    const int64_t ntn = (N + BN - 1) / BN, nkt = K / SB;
    const int64_t pieces = E * ntn * nkt * BN * (SB / 16);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pieces; i += (int64_t)gridDim.x * blockDim.x) {
        const int p = (int)(i % (SB / 16));  // position of the piece in its row
        const int64_t rowi = i / (SB / 16);
        const int r = (int)(rowi % BN);
        const int64_t blk = rowi / BN;  // (e * ntn + nt) * nkt + kt
        const int64_t kt = blk % nkt, ent = blk / nkt;
        const int64_t nt = ent % ntn, e = ent / ntn;
        const int64_t n = nt * BN + r;
        // the position holds the global piece whose swizzled position it is
        const int c = swz_chunk<SB>(r, p);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n < N) v = *reinterpret_cast<const uint4*>(b + (e * N + n) * K + kt * SB + c * 16);
        *reinterpret_cast<uint4*>(out + i * 16) = v;
    }
}

// 256 x 384 or 256 x 256 FP8 tiles (both give the same bits).  Measured on
// the prefill shape (N = 1536, K = 4096) from 8k to 64k rows, dense and
// ragged: a 256 x 384 tile takes ~1.4x as long as a 256 x 256 one (1.5x the
// work at a sixth fewer operand bytes per FLOP), and a persistent round costs
// about as much whether its tiles are whole or split, so the wider tile pays
// when its rounds, weighted 1.4, are fewer (dense 16k rows 0.74x, ragged 64k
// 0.88x; dense 8k 1.26x, ragged 8k over 128 experts 1.06x).  The host does
// not see the group sizes: the M tiles are estimated as T / 256 plus the
// padding of each group, half a tile for groups of 256+ rows on average and
// up to a whole one as the average falls to none (Zipf-routed 8k-64k rows
// over 32 and 128 experts: estimates 48-320 against 48-314).  The wide tile
// needs rows of c on 16 bytes (its two-pass epilogue) and is not used where
// it pads N further than 256 columns do.  MXG_FP8_TILE=256x384 / 256x256
// overrides the choice (tuning, tests); other values are ignored.
bool wide_fp8_pays(const GemmProblem& p) {
    if (p.N % 8 != 0) return false;
    if (const char* v = getenv("MXG_FP8_TILE")) {
        if (strcmp(v, "256x384") == 0) return true;
        if (strcmp(v, "256x256") == 0) return false;
    }
    const int64_t ntn_w = (p.N + 383) / 384, ntn_s = (p.N + 255) / 256;
    if (ntn_w * 384 > ntn_s * 256) return false;
    const int64_t groups = p.G < p.T ? p.G : p.T;
    if (groups <= 0) return false;
    const int64_t avg = p.T / groups;
    const int64_t pad = 128 + (avg < 256 ? 128 - avg / 2 : 0);  // 256ths of a tile per group
    const int64_t mt = p.T / 256 + groups * pad / 256;
    const int cus_q = device_cus();
    const int64_t cus = cus_q > 0 ? cus_q : 256;
    const int64_t rounds_w = (mt * ntn_w + cus - 1) / cus, rounds_s = (mt * ntn_s + cus - 1) / cus;
    return 14 * rounds_w < 10 * rounds_s;
}

// Rows per group that decide the regime: the average over non-empty groups,
// moved halfway to the optional host hint (largest group) when that is larger
// (the hint can only move a problem to the larger tile).
int64_t regime_rows(const GemmProblem& p) {
    const int64_t groups = p.G < p.T ? p.G : p.T;
    const int64_t avg_rows = groups > 0 ? p.T / groups : p.T;
    return p.max_rows_hint > avg_rows ? (avg_rows + p.max_rows_hint) / 2 : avg_rows;
}

}  // namespace

// The FP8 rowwise tile launch_grouped_gemm runs: 384 or 256 (256-row tiles of
// that many columns), 32 (the decode-regime 32 x 256 tile), 0 for anything
// else (other formats, the fused epilogue, prepared weights with K % 64 != 0).
int fp8_tile_choice(const GemmProblem& p) {
    if (p.fmt != 0 || p.yq != nullptr) return 0;
    if (p.b_prepared) return p.K % 64 != 0 ? 0 : wide_fp8_pays(p) ? 384 : 256;
    if (regime_rows(p) < 128) return 32;
    return p.K % 64 == 0 && wide_fp8_pays(p) ? 384 : 256;
}

namespace {

template <int FMT, bool SWIGLU>
hipError_t launch_fmt(const GemmProblem& p, hipStream_t stream) {
    if constexpr (FMT == 3) {
        // NVFP4: the 128 x 256 tile with LDS-staged scales (K a multiple of 512)
        return launch_tile<TileLargeMxKA, FMT, SWIGLU, true>(p, stream, kBandMx);
    } else {
        if constexpr (FMT == 0) {
            // 256 x 384 where it pays, else 256 x 256 (whole 64-byte stages
            // in the four-slot pipeline, or 128-byte stages with a K tail);
            // few rows per group: the 32 x 256 decode tile
            const int choice = fp8_tile_choice(p);
            if (choice == 384) return launch_tile<TileWideFp8, FMT, SWIGLU, true>(p, stream, kBandLarge);
            if (choice == 256)
                return p.K % 64 == 0 ? launch_tile<TileLargeFp8, FMT, SWIGLU, true>(p, stream, kBandLarge)
                                     : launch_tile<TileLargeFp8Tail, FMT, SWIGLU, false>(p, stream, kBandLarge);
            return launch_tile<TileSmallFp8, FMT, SWIGLU, false>(p, stream, kBandNOuter);
        } else {
            if (regime_rows(p) >= 128) {
                // whole 128-byte stages and whole 32-byte scale chunks (LDS-staged scales)
                const int64_t groups = p.G < p.T ? p.G : p.T;
                const int64_t avg_rows = groups > 0 ? p.T / groups : p.T;
                const bool ka = p.K % 1024 == 0;
                if (ka && avg_rows >= kTallRows)
                    return launch_tile<TileLargeMxKA8, FMT, SWIGLU, true>(p, stream, kBandLarge);
                return ka ? launch_tile<TileMx192, FMT, SWIGLU, true>(p, stream, kBandMx)
                          : launch_tile<TileLargeMx, FMT, SWIGLU, false>(p, stream, kBandMx);
            }
            return launch_tile<TileSmall, FMT, SWIGLU, false>(p, stream, kBandNOuter);
        }
    }
}

}  // namespace

namespace gemm {

int device_cus() {
    static thread_local int cached_device = -1, cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (cached_device != dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached_device = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

GemmArgs make_args(const GemmProblem& p, int BM, int BN, int mband, int per_cu, int64_t* grid) {
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
    a.row_bytes = (p.fmt == 2 || p.fmt == 3) ? p.K / 2 : p.K;
    a.ntiles_n = (int)((p.N + BN - 1) / BN);
    a.mband = mband > 0 ? mband : 1;
    a.es = p.es;
    a.rs = static_cast<const uint16_t*>(p.rs);
    a.ysf = p.ysf;
    a.asoff = p.asoff;
    a.as_rows = p.as_rows;
    // Upper bound on M tiles: each non-empty group adds at most one partial tile.
    const int64_t groups_nonempty = p.G < p.T ? p.G : p.T;
    const int64_t mtiles_bound = p.T / BM + groups_nonempty;
    const int64_t tiles_bound = mtiles_bound * a.ntiles_n;
    const int cus = device_cus();
    int64_t g = (int64_t)(cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
    *grid = g < tiles_bound ? g : tiles_bound;
    return a;
}

}  // namespace gemm

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream) {
    const bool swiglu = p.yq != nullptr;
    if (p.b_prepared) {
        // the ring that reads prepared weights, whatever the rows per group
        const int choice = fp8_tile_choice(p);
        if (choice == 384) return launch_tile<TileWideFp8Prep, 0, false, true>(p, stream, kBandLarge);
        if (choice == 256) return launch_tile<TileLargeFp8Prep, 0, false, true>(p, stream, kBandLarge);
        return hipErrorInvalidValue;
    }
    switch (p.fmt) {
        case 0:
            return launch_fmt<0, false>(p, stream);
        case 1:
            return swiglu ? launch_fmt<1, true>(p, stream) : launch_fmt<1, false>(p, stream);
        case 2:
            return swiglu ? launch_fmt<2, true>(p, stream) : launch_fmt<2, false>(p, stream);
        case 3:
            return swiglu ? launch_fmt<3, true>(p, stream) : launch_fmt<3, false>(p, stream);
        default:
            return hipErrorInvalidValue;
    }
}

int64_t prepared_weights_bytes(int64_t E, int64_t N, int64_t K) {
    constexpr int BN = kPrepRows;
    return E * ((N + BN - 1) / BN) * BN * K;
}

hipError_t launch_prepare_weights(const void* b, int64_t E, int64_t N, int64_t K, void* out, hipStream_t stream) {
    if (K % TileLargeFp8Prep::kSB != 0) return hipErrorInvalidValue;
    const int64_t pieces = prepared_weights_bytes(E, N, K) / 16;
    if (pieces <= 0) return hipSuccess;
    const int cus = gemm::device_cus();
    int64_t blocks = (pieces + 255) / 256;
    const int64_t cap = (int64_t)(cus > 0 ? cus : 256) * 8;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(prepare_weights_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(b), E, N, K, static_cast<uint8_t*>(out));
    return hipGetLastError();
}

}  // namespace mxg
