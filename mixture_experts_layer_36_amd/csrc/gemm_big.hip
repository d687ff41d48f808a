// Prefill-shaped grouped GEMM for gfx950: 256 x BN block tiles fed by
// direct-to-LDS loads through a 4-stage pipeline.
//
// Experts run as grouped GEMMs over their expert-contiguous rows ("Tensor vs
// Expert vs Data Parallelism for MoE Serving", section "Deeper Analysis",
// Figure 2); in the large-batch regime each expert sees enough rows for the
// GEMM to be compute-bound (same page, section "Why sparsity demands a large
// batch").  This kernel is built for that regime:
//   * block tile 256 activation rows x BN weight rows (BN = 256 or 128),
//     BK = 32, four wavefronts in a 2 x 2 grid, so each wavefront owns a
//     128 x (BN/2) tile as 16x16 blocks: per stage 64 (or 32)
//     v_mfma_f32_16x16x32_bf16 on 16 (or 12) 128-bit LDS fragment reads,
//     with the accumulators in AGPRs.  The 16x16x32 form does the same work
//     per cycle as 32x32x16 but moves a quarter of the accumulator registers
//     per MFMA: the GEMM-shaped MFMA loop alone on random bf16 operands
//     sustains 2086 TFLOP/s against 1842 (MI355X, same power limit);
//   * global -> LDS with global_load_lds_dwordx4 (no VGPR staging) into a
//     4-deep ring of 32 KB stages; each wave waits only for its own loads of
//     the next stage (vmcnt) and a bare s_barrier publishes them, so later
//     stages stay in flight;
//   * a stage is one k32 step: its MFMAs run on fragments read during the
//     previous stage (two fragment sets), laid out as groups of MFMAs, each
//     followed by at most one direct load and a share of the next stage's
//     fragment reads, fenced by sched_barrier so the compiler keeps that
//     order: left to itself it sank a step's loads past all of its fragment
//     reads and issued them in a burst beside the barrier.  The barrier
//     comes two groups into the stage, after which the stage's buffer is
//     free and is refilled with the stage four ahead: three stages of lead
//     for every load (against the 32x32x16 two-step schedule: Qwen-shaped
//     fp8-weight layer gate-up 1406 -> 1305 us and down 837 -> 776 us,
//     Mixtral-shaped gate-up 1608 -> 1526 us and down 782 -> 721 us,
//     DeepSeek-V3-shaped down 3758 -> 3688 us; its gate-up, at the power
//     limit and on the load path, unchanged);
//   * an expert's last tile with at most 128 (64) rows runs a half-height
//     (quarter-height) layout: all four wavefronts on those rows, each with
//     half the weight rows, so a short tail loads and multiplies only its
//     own rows rather than a whole tile's;
//   * tiles that remain after the last full wave of tiles (one tile per
//     compute unit) are split along K into pieces that fill that wave; each
//     piece stores its raw fp32 accumulators and a fixup kernel adds the
//     pieces in order and applies the epilogue (many blocks per split tile,
//     one 4-column run per work unit), so the result is deterministic
//     (the down projection of a Mixtral-shaped layer has 2.25 waves of
//     tiles, so without this its last wave would run a quarter full);
//   * with the fp8 dispatch payload as activations and E4M3 weights, the
//     gate-up GEMM runs both operands in fp8 on the block-scaled MFMA
//     (big_tile_fp8 below);
//   * LDS rows of BK elements with 16-byte chunks XOR-swizzled by row
//     ((r >> 2) & 3 for 64-byte rows, (r ^ (r >> 3)) & 7 for 128-byte rows;
//     fp8 weight rows of 32 bytes: (r >> 3) & 1): a 128-bit read is served
//     16 lanes at a time on gfx950's 64 banks, and the 16 lanes of one
//     fragment read take one chunk of 16 consecutive rows, which the
//     swizzle spreads over all banks.  A direct load writes 64 consecutive
//     16-byte slots, so each lane fetches the global chunk that belongs in
//     its slot;
//   * operands row-major or K-blocked (32-column planes of [rows][32]: the
//     expert weights when packed, h between the two routed GEMMs, x_perm for
//     wide experts): K-blocked, a stage's slice of a tile's consecutive rows
//     is one contiguous run, so a 1 KB direct load covers 8 whole cache
//     lines instead of 16 half lines;
//   * every buffer descriptor is built from block-uniform values stated
//     uniform (readfirstlane): otherwise the compiler cannot prove a base
//     computed on the vector unit uniform and wraps each load through it in a
//     loop over distinct lane values;
//   * with a tile table, a schedule kernel resolves every block's tile ahead
//     of the launch (big_sched_kernel), so a block starts from one 32-byte
//     record rather than three dependent loads and the integer divisions of
//     the grouped order and split plan (DeepSeek-V3-shaped layer -0.6%);
//   * the tile's outputs (h planes, y rows) go out with non-temporal stores:
//     each is read once, by a later launch, and kept out of L2 they leave it
//     to the operand tiles the blocks of an XCD share.
#include <atomic>

#include "gemm_common.hpp"

namespace moe {
namespace {

#ifndef MOE_BIG_WN
#define MOE_BIG_WN 2
#endif
constexpr int BM = 256, BK = 32, STAGES = 4;
constexpr int CH = BK / 8;        // 16-byte chunks per LDS row

// Tile layouts, LAY = 0, 1, 2.  Full (0): WN wavefronts along the weight
// rows, 2 along the 256 activation rows, each wave 128 activation rows x RW
// weight rows.  Half (1, tiles of at most 128 rows): all 2*WN wavefronts on
// the 128 activation rows, each with RW/2 weight rows.  Quarter (2, at most
// 64 rows): the same weight split over 64 activation rows.  The LDS ring is
// the same; a shorter layout loads and multiplies only its rows.
// BH: the edge of the MFMA blocks -- 16 for the bf16-operand tiles
// (16x16x32 MFMAs), 32 for the fp8 x fp8 tiles (32x32x64).
template <int BN, int WN, int LAY, int BH = 32>
struct BigCfg {
  static constexpr int NTHR = 128 * WN;
  static constexpr int RW = BN / WN;                 // weight rows per wave column (full layout)
  static constexpr int TA = (LAY == 2 ? 64 : 128) / BH;  // activation blocks per wave
  static constexpr int TW = (LAY ? RW / 2 : RW) / BH;    // weight blocks per wave
  static constexpr int NACC = BH * BH / 64;          // accumulator floats per lane and block
  static constexpr int RUNS = NACC / 4;              // runs of 4 output columns per lane and block
  static constexpr int A_ROWS = BM >> LAY;           // activation rows loaded
  static_assert(TW >= 1 && LAY >= 0 && LAY <= 2 && (BH == 16 || BH == 32), "layout");
};
template <int BH>
struct AccOf;
template <>
struct AccOf<16> {
  using T = f32x4;
};
template <>
struct AccOf<32> {
  using T = f32x16;
};

// The layout of a tile with `nrows` rows.
__device__ __forceinline__ int tile_layout(int nrows) { return nrows <= BM / 4 ? 2 : nrows <= BM / 2 ? 1 : 0; }

// Stage bytes and 16-byte loads per thread.  bf16 weight rows are BK * 2 = 64
// bytes (4 chunks); fp8 (E4M3) rows are 32 bytes (2 chunks), half the traffic.
template <int BN, int WN, int LAY, int WDT>
struct BigMem {
  static constexpr int NTHR = 128 * WN;
  static constexpr int WB = (WDT == GD_FP8) ? 1 : 2;  // weight bytes per element
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BN * BK * WB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS");
  static constexpr int A_LOADS = BigCfg<BN, WN, LAY>::A_ROWS * BK * 2 / 16 / NTHR;
  static constexpr int B_LOADS = B_BYTES / 16 / NTHR;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "layout");
};

// fp8 weight rows in LDS: 32 bytes = two 16-byte chunks, chunk c of row r at
// c ^ ((r >> 3) & 1), so the 16 rows one 128-bit read pass serves cover all
// 64 banks once.
[[maybe_unused]] __device__ __forceinline__ int f8_off(int r, int c) { return r * 32 + ((c ^ ((r >> 3) & 1)) << 4); }

// Eight OCP E4M3 codes -> eight bf16, exactly (every E4M3 value is a bf16
// value): gfx950's packed scaled conversion, two codes per instruction, with
// a scale of 1.0 (exhaustively equal to the f32-path conversion's upper
// halves for all code pairs); half the instructions of converting to f32 and
// packing the upper halves.
[[maybe_unused]] __device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS weight row of a wave's block i, its first activation row and the first
// output column of its blocks (relative to the tile's first column).  SwiGLU
// tiles hold, per wave column of the full layout, RW/2 rows of W1 followed
// by the same columns of W3, and a wave's blocks i < TW/2 are W1 (u), the
// blocks i + TW/2 the matching W3 (v).
template <int BN, int WN, int LAY, int EPI, int BH>
__device__ __forceinline__ int wave_wrow(int wave, int i) {
  using C = BigCfg<BN, WN, LAY, BH>;
  if (!LAY) return (wave % WN) * C::RW + i * BH;
  if (EPI != EPI_SWIGLU) return wave * (C::RW / 2) + i * BH;
  const int slab = wave >> 1, sub = wave & 1;
  return i < C::TW / 2 ? slab * C::RW + sub * (C::RW / 4) + i * BH
                       : slab * C::RW + C::RW / 2 + sub * (C::RW / 4) + (i - C::TW / 2) * BH;
}
template <int BN, int WN, int LAY>
__device__ __forceinline__ int wave_arow(int wave) {
  return LAY ? 0 : (wave / WN) * 128;
}
template <int BN, int WN, int LAY, int EPI>
__device__ __forceinline__ int wave_col(int wave) {
  using C = BigCfg<BN, WN, LAY>;
  if (!LAY) return (wave % WN) * (EPI == EPI_SWIGLU ? C::RW / 2 : C::RW);
  if (EPI != EPI_SWIGLU) return wave * (C::RW / 2);
  return (wave >> 1) * (C::RW / 2) + (wave & 1) * (C::RW / 4);
}

// Chunk swizzle: the rows read by one fragment load (32 consecutive rows, one
// logical chunk) spread over distinct LDS bank groups.
__device__ __forceinline__ int swz(int r) {
  return CH == 4 ? ((r >> 2) & 3) : ((r ^ (r >> 3)) & 7);
}
// element offset of (row r, logical 16-byte chunk c) in a BK-wide tile
[[maybe_unused]] __device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ swz(r)) << 3); }


template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
[[maybe_unused]] __device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// f(IC<I>{}) for I = B .. E-1, each with I a constant expression.
template <int V>
struct IC {
  static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}


// Split plan over R real tiles on n_cu compute units: the first `full`
// tiles run whole; each of the `rem` others is split into `s` K-pieces
// (s >= 2, each piece >= 8 stages of the kt_plan stages, rem * s <= slots).
struct SplitPlan {
  int full, rem, s;
};
__device__ __forceinline__ SplitPlan split_plan(int R, int kt_plan, int n_cu, int slots) {
  SplitPlan p{R, 0, 1};
  if (slots <= 0 || R <= 0 || n_cu <= 0) return p;
  const int w = R / n_cu, r = R - w * n_cu;
  if (r == 0) return p;
  const int s = min(min(n_cu / r, kt_plan / 8), slots / r);
  if (s < 2) return p;
  p.full = w * n_cu;
  p.rem = r;
  p.s = s;
  return p;
}

// What one block computes: tile (mt, nt), k-stages [k0, k1) of its segment's
// KT, and the partial slot of a split piece (-1: the whole tile).
struct Work {
  int mt, nt, k0num, slot, s;
};
// Blocks are dealt round-robin to the 8 XCDs (block b on XCD b % 8).  Whole
// tiles come first, an equal share per XCD (xcd_tile: whole groups in turn,
// so the blocks an XCD runs at once share operands in its L2); the split
// pieces follow, again an equal share per XCD, so they all run in the last
// wave.
[[maybe_unused]] __device__ __forceinline__ bool big_work(const GemmArgs& a, int n_tiles, int kt_plan, int n_cu,
                                         int BMv, Work& w, int bid) {
  const int m_real = real_mtiles(a, BMv);
  const int R = m_real * n_tiles;
  const SplitPlan p = split_plan(R, kt_plan, n_cu, a.partial ? a.partial_slots : 0);
  const int x = bid & 7, i = bid >> 3;
  int L;
  w.slot = -1;
  w.k0num = 0;
  w.s = 1;
  if (p.rem > 0) {
    const int f8 = p.full >> 3, Q = p.rem * p.s, q = (Q + 7) >> 3;
    if (i < f8) {
      if (!xcd_tile(x, i, p.full, n_tiles, L)) return false;
    } else {
      const int j = i - f8, pi = x * q + j;
      if (j >= q || pi >= Q) return false;
      L = p.full + pi / p.s;
      w.k0num = pi % p.s;
      w.slot = pi;
      w.s = p.s;
    }
  } else {
    if (!xcd_tile(x, i, R, n_tiles, L)) return false;
  }
  tile_coords(L, m_real, n_tiles, w.mt, w.nt);
  return true;
}

// Rows per m-tile: 256, or a.m_tile (128) for a launch without a tile table
// (the router logits, whose plan picks 128-row tiles where 256-row ones would
// need short K ranges to fill the GPU).
__host__ __device__ __forceinline__ int m_tile_rows(const GemmArgs& a) {
  return (a.tile_table == nullptr && a.m_tile == BM / 2) ? BM / 2 : BM;
}

// Block bid's tile, K-piece and rows: from its record when a schedule kernel
// wrote one for every block of the launch (gridDim.x <= sched_cap), else
// derived here.  A record holds mt, nt, k0num, slot, s, e, row0, nrows (mt < 0:
// no work); one that does not fit the segment it names is treated as empty.
[[maybe_unused]] __device__ __forceinline__ bool big_block(const GemmArgs& a, int n_tiles, int kt_plan, int n_cu,
                                                           int BMv, int ncols, Work& wk, TileInfo& ti, Seg& sg) {
  if (a.sched != nullptr && a.tile_table != nullptr && (int)gridDim.x <= a.sched_cap) {
    const int4* r = (const int4*)(a.sched + (size_t)blockIdx.x * kSchedInts);
    const int4 r0 = r[0], r1 = r[1];
    wk.mt = __builtin_amdgcn_readfirstlane(r0.x);
    wk.nt = __builtin_amdgcn_readfirstlane(r0.y);
    wk.k0num = __builtin_amdgcn_readfirstlane(r0.z);
    wk.slot = __builtin_amdgcn_readfirstlane(r0.w);
    wk.s = __builtin_amdgcn_readfirstlane(r1.x);
    ti.e = __builtin_amdgcn_readfirstlane(r1.y);
    ti.row0 = __builtin_amdgcn_readfirstlane(r1.z);
    ti.nrows = __builtin_amdgcn_readfirstlane(r1.w);
    if (wk.mt < 0 || ti.e < 0 || ti.e > a.E || ti.nrows <= 0 || ti.nrows > BMv || ti.row0 < 0) return false;
    if (ti.row0 + ti.nrows > (ti.e == a.E ? a.sh_rows : a.rows)) return false;
    tile_seg(a, ti, sg);
    return wk.nt * ncols < sg.N;
  }
  if (!big_work(a, n_tiles, kt_plan, n_cu, BMv, wk, blockIdx.x)) return false;
  if (!tile_info(a, wk.mt, BMv, ti, sg)) return false;
  return wk.nt * ncols < sg.N;
}

// One thread per block of the GEMM launch: the record big_block reads.
__global__ __launch_bounds__(256) void big_sched_kernel(GemmArgs a, int n_tiles, int kt_plan, int n_cu, int BMv,
                                                        int ncols, int nb) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  Work wk;
  TileInfo ti;
  Seg sg;
  int4 r0 = make_int4(-1, 0, 0, -1), r1 = make_int4(1, 0, 0, 0);
  if (big_work(a, n_tiles, kt_plan, n_cu, BMv, wk, b) && tile_info(a, wk.mt, BMv, ti, sg) && wk.nt * ncols < sg.N) {
    r0 = make_int4(wk.mt, wk.nt, wk.k0num, wk.slot);
    r1 = make_int4(wk.s, ti.e, ti.row0, ti.nrows);
  }
  int4* r = (int4*)(a.sched + (size_t)b * kSchedInts);
  r[0] = r0;
  r[1] = r1;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Buffer descriptor word 3 for raw 32-bit-format buffers on gfx9-family GPUs.
[[maybe_unused]] constexpr int kBufferFlags = 0x00020000;

// A buffer descriptor from block-uniform values, stated uniform: a base
// whose 64-bit offset was computed on the vector unit otherwise leaves the
// compiler unsure, and it wraps every load through the descriptor in a
// loop over distinct lane values.
[[maybe_unused]] __device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// Output columns of a tile and the LDS bytes of its staged copy.
template <int BN, int EPI>
struct OutTile {
  static constexpr int COLS = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  static constexpr int ROW_BYTES = COLS * 2;  // bf16
  static constexpr int CPR = COLS / 8;        // 16-byte chunks per row
  static constexpr int BYTES = BM * ROW_BYTES;
  static_assert(CPR >= 16 && (CPR & (CPR - 1)) == 0, "chunk swizzle");
};

#if defined(__HIP_DEVICE_COMPILE__)
// End of a tile with the SwiGLU or plain-store epilogue (bf16 out), or of a
// K-piece of a split tile.  In MFMA block (i, j) of edge BH, lane l holds
// output columns i*BH + g*8 + (l/BH)*4 + q (q = 0..3, run g < BH*BH/256)
// of activation row j*BH + l % BH: runs of 4 consecutive columns.
//   * A whole tile goes out through LDS: each wave writes its runs into a
//     row-major copy of the tile, 16-byte chunk c of row r at c ^ (r & 15)
//     (the rows one write touches spread over the banks); then the block
//     stores whole rows with 16-byte writes, so one wave instruction covers
//     2-4 full row runs rather than one run per lane.  The operand ring is
//     dead by then: every wave has read its last fragments.
//   * A piece stores its raw accumulators to its partial slot, register-major
//     so that each 16-byte store of a wave is contiguous.
// Both are handled block by block in one pass.  lds_sc: the tile's fp8
// channel scales, staged in LDS by the prologue (stage_scales): BN of them
// (SwiGLU: BN/2 of W1, then BN/2 of W3).
template <int BN, int WN, int EPI, int LAY, int WDT, int BH>
__device__ __forceinline__ void finish_tile(
    const GemmArgs& a, const TileInfo& ti, const Seg& sg,
    typename AccOf<BH>::T (&acc)[BigCfg<BN, WN, LAY, BH>::TW][BigCfg<BN, WN, LAY, BH>::TA], int ncol0,
    char* lds, int slot, const float* lds_sc) {
  using C = BigCfg<BN, WN, LAY, BH>;
  using O = OutTile<BN, EPI>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int arow = wave_arow<BN, WN, LAY>(wave), wcol = wave_col<BN, WN, LAY, EPI>(wave);
  const bool piece = slot >= 0;
  const bool scaled = WDT == GD_FP8 && sg.s0 != nullptr && !piece;
  float4* P = (float4*)(a.partial + (size_t)(piece ? slot : 0) * (kPartialSlotBytes / 4));
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  barrier_only();
  auto put = [&](int lrow, int lcol, float v0, float v1, float v2, float v3) {
    u32x2 o;
    o[0] = pack_bf16x2(v0, v1);
    o[1] = pack_bf16x2(v2, v3);
    *(u32x2*)(lds + lrow * O::ROW_BYTES + (((lcol >> 3) ^ (lrow & 15)) << 4) + (lcol & 7) * 2) = o;
  };
  auto raw = [&](int i, int j, int g) {
    P[((i * C::TA + j) * C::RUNS + g) * C::NTHR + tid] =
        make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
  };
  constexpr int NB = (EPI == EPI_SWIGLU) ? C::TW / 2 : C::TW;
#pragma unroll
  // Run by run (4 columns of BH activation rows per lane and block): only
  // that run's fp8 channel scales stay live, which keeps the fp8-weight
  // epilogue's register spills down.
  for (int i = 0; i < NB; ++i) {
#pragma unroll
    for (int g = 0; g < C::RUNS; ++g) {
      const int lcol = wcol + i * BH + g * 8 + (lane / BH) * 4;
      float4 su = make_float4(1.f, 1.f, 1.f, 1.f), sv = su;
      if (scaled) {
        su = *(const float4*)(lds_sc + lcol);
        if (EPI == EPI_SWIGLU) sv = *(const float4*)(lds_sc + BN / 2 + lcol);
      }
      const float s4u[4] = {su.x, su.y, su.z, su.w}, s4v[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int j = 0; j < C::TA; ++j) {
        if (piece) {
          raw(i, j, g);
          if (EPI == EPI_SWIGLU) raw(i + C::TW / 2, j, g);
        }
        // a piece also fills the LDS copy (never stored): with no second
        // path the compiler keeps the accumulators in AGPRs
        const int lrow = arow + j * BH + lane % BH;
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float u = acc[i][j][g * 4 + q] * s4u[q];
          if (EPI == EPI_SWIGLU) {
            const float v = acc[i + C::TW / 2][j][g * 4 + q] * s4v[q];
            o[q] = silu(u) * v;
          } else {
            o[q] = u;
          }
        }
        put(lrow, lcol, o[0], o[1], o[2], o[3]);
      }
      // one run at a time: the accumulators leave the AGPRs as needed
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (piece) return;
  __builtin_amdgcn_s_waitcnt(0xc07f);
  barrier_only();
  const int rows = ti.nrows;
  if (sg.c_prows) {
    // K-blocked C: the tile's 32-column planes in turn, each a contiguous run
    // of rows x 64 bytes (4 chunks per row): chunk q of a plane's run is row
    // q / 4, chunk q % 4, at element 8 q of the run.  Non-temporal stores:
    // h is read once, by the next GEMM, long after the tile, so its lines
    // need not displace the operand tiles the blocks of an XCD share in L2
    // (DeepSeek-V3-shaped layer -0.2%, Qwen-shaped gate-up -1.2%, Mixtral-
    // shaped layer -0.5%)
#pragma unroll
    for (int p = 0; p < O::CPR / 4; ++p) {
      if (ncol0 + p * 32 >= sg.N) break;
      uint16_t* run = (uint16_t*)sg.C + ((size_t)(ncol0 / 32 + p) * sg.c_prows + ti.row0) * 32;
      for (int q = tid; q < rows * 4; q += C::NTHR) {
        const int r = q >> 2, ch = p * 4 + (q & 3);
        __builtin_nontemporal_store(*(const u32x4*)(lds + r * O::ROW_BYTES + ((ch ^ (r & 15)) << 4)),
                                    (u32x4*)(run + q * 8));
      }
    }
    return;
  }
  // Row-major C (the down projection's y rows): non-temporal as well.  The
  // combine reads each row once, a whole launch later; kept out of L2 they
  // leave it to the operand tiles (DeepSeek-V3-shaped down GEMM 3780 -> 3716
  // us, Qwen-shaped 790 -> 778 us, the combine unchanged)
  for (int u = tid; u < rows * O::CPR; u += C::NTHR) {
    const int r = u / O::CPR, ch = u % O::CPR;
    const u32x4 v = *(const u32x4*)(lds + r * O::ROW_BYTES + ((ch ^ (r & 15)) << 4));
    if (ncol0 + ch * 8 < sg.N)
      __builtin_nontemporal_store(v, (u32x4*)((uint16_t*)sg.C + (size_t)(ti.row0 + r) * sg.N + ncol0 + ch * 8));
  }
}

// The fp8 channel scales of a whole tile's columns into LDS (lds_sc, BN
// floats; SwiGLU: BN/2 of W1 then BN/2 of W3), one dword direct load per
// lane, issued before the tile's first stage so the prologue's wait for
// stage 0 covers it; columns past N read 0 (the descriptor's bound).  The
// epilogue then reads them from LDS instead of waiting on global loads.
template <int BN, int EPI, int NTHR>
__device__ __forceinline__ void stage_scales(const Seg& sg, int ncol0, float* lds_sc, int wave) {
  constexpr int HALF = BN / 2;
  if (wave * 64 >= BN) return;
  const bool w3 = EPI == EPI_SWIGLU && wave * 64 >= HALF;
  const float* src = (w3 ? sg.s1 : sg.s0) + ncol0;
  const __amdgpu_buffer_rsrc_t r = uniform_rsrc(src, (sg.N - ncol0) * 4);
  const int c0 = (EPI == EPI_SWIGLU && w3) ? wave * 64 - HALF : wave * 64;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds_sc + wave * 64), 4,
                                           (uint32_t)((c0 + (int)(threadIdx.x & 63)) * 4), 0, 0, 0);
  static_assert(BN <= NTHR, "one scale per thread");
}

// Pipeline of the bf16-operand tiles: per stage (32 k values) NG groups,
// GB of them before the stage's barrier; the reads of the next stage's
// fragments are spread over groups GB..NG-1.
#ifndef MOE_BIG_GB
#define MOE_BIG_GB 2
#endif
constexpr int kNG = 16, kGB = MOE_BIG_GB;
// The order of a stage's fragment reads (position -> fragment; weight blocks
// 0..TW-1, activation blocks TW..).  bf16: the order the MFMAs (weight-block
// major) first use them, w0, every x, then w1 ..  fp8 weights (raw bytes,
// widened groups later): two weight blocks, then activation and weight
// blocks alternately (w0 w1 x0 w2 x1 w3 ..), so every weight block lands
// well before its widening.
template <int TW, int TA, int WDT>
constexpr int frag_order(int pos) {
  if (WDT == GD_FP8) {
    int w = 0, x = 0;
    for (int p = 0;; ++p) {
      const bool take_w = w < TW && (p < 2 || x >= TA || (p % 2 == 1));
      const int q = take_w ? w++ : TW + x++;
      if (p == pos) return q;
    }
  }
  return pos == 0 ? 0 : pos <= TA ? TW + pos - 1 : pos - TA;
}
// The first read position of group g (GB <= g <= NG) of NDS reads.
template <int NDS>
constexpr int read_pos(int g) {
  return (g - kGB) * NDS / (kNG - kGB);
}
// The group that reads fragment q, and (fp8 weights) the group that widens
// weight block i: one of the last TW groups, at least two groups after its
// read; NG or more: after the groups.
template <int TW, int TA, int WDT>
constexpr int read_group(int q) {
  int pos = 0;
  while (frag_order<TW, TA, WDT>(pos) != q) ++pos;
  int g = kGB;
  while (read_pos<TW + TA>(g + 1) <= pos) ++g;
  return g;
}
template <int TW, int TA, int WDT>
constexpr int widen_group(int i) {
  const int r = read_group<TW, TA, WDT>(i) + 2, l = kNG - TW + i;
  return r > l ? r : l;
}

// Wide A (64-column planes, a K-blocked A only): swizzle of a 128-byte LDS
// row, chunk c of row r at c ^ swz8(r): the 16 rows of one fragment read
// (one chunk each) cover all 64 banks.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// One tile (or K-piece of a tile) in the full, half or quarter layout.
// WIDE: A in 64-column planes (GemmArgs::a_blk == 2).  Each A load then
// brings a row's 128 bytes, the A of two consecutive stages, so the ring
// holds A as two pair buffers (32 KB each: row r's bytes 0-63 the even
// stage, 64-127 the odd one) beside four B buffers; the same 128 KB.
template <int BN, int WN, int EPI, int LAY, int WDT, bool WIDE>
__device__ __forceinline__ void big_tile(const GemmArgs& a, const TileInfo& ti, const Seg& sg, const Work& wk,
                                         int ncol0, char* lds, float* lds_sc) {
  using C = BigCfg<BN, WN, LAY, 16>;
  using M = BigMem<BN, WN, LAY, WDT>;
  constexpr int LA = WIDE ? 2 * M::A_LOADS : M::A_LOADS;  // A loads of one refill (WIDE: a pair of stages)
  constexpr int A_PAIR = BM * 128;                         // LDS bytes of a pair's A (WIDE)
  static_assert(!WIDE || 2 * A_PAIR + STAGES * M::B_BYTES <= STAGES * M::STAGE_BYTES, "wide ring");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: SGPR arithmetic
  const int K = sg.K;
  // this block's k-stages of the segment: all, piece k0num of s, or (router
  // logits) the blockIdx.y-th of ksplit ranges
  const int KT_all = K / BK;
  const int np = wk.s * a.ksplit, pi = wk.k0num * a.ksplit + (int)blockIdx.y;
  // WIDE: K a multiple of 64 and pieces start on even stages (whole pairs)
  const int kt0 = WIDE ? 2 * (pi * (KT_all / 2) / np) : pi * KT_all / np;
  const int kt1 = WIDE ? 2 * ((pi + 1) * (KT_all / 2) / np) : (pi + 1) * KT_all / np;

  // Direct loads go through buffer resources: a block-uniform descriptor
  // (SGPRs) per operand, a 32-bit per-lane byte offset fixed across stages
  // and the stage's k offset as the scalar offset, so each load is a single
  // buffer_load_dwordx4 ... lds with no per-stage address arithmetic.  The
  // descriptor's size bounds every access to the tile's own rows.  Slot s of
  // a stage's tile is row s / CH, physical chunk s % CH, which holds logical
  // chunk (s % CH) ^ swz(row).
  const int KT = kt1 - kt0;
  // With a row map (fused dispatch gather) the descriptor spans all of A and
  // each lane's offset starts at its row's A row.  A K-blocked A (planes of
  // a_prows rows, no row map) spans all planes: a lane's offset is its row's
  // 64 bytes in plane 0 and a stage adds its plane, so a load of the stage's
  // 32-column slice reads consecutive rows as one contiguous run.
  // WIDE: planes of 64 columns, a lane's offset its row's 128 bytes in plane
  // 0 (slot s of a pair's tile is row s / 8, physical chunk s % 8) and a
  // refill of a pair adds its plane.
  constexpr int APW = WIDE ? 64 : BK;  // A plane width (columns)
  const int a_plane = sg.a_prows * APW * 2;  // 0: row-major
  const int a_step = a_plane ? a_plane : BK * 2;  // bytes from one refill's slice to the next
  const __amdgpu_buffer_rsrc_t a_rsrc =
      a_plane ? uniform_rsrc(sg.A, (K / APW) * a_plane)
      : sg.amap ? uniform_rsrc(sg.A, a.a_map_rows * K * 2)
                : uniform_rsrc(sg.A + (size_t)ti.row0 * K * 2, ti.nrows * K * 2);
  uint32_t a_off[LA];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int s = (wave * LA + j) * 64 + lane;
    const int r = WIDE ? s / 8 : s / CH, c = WIDE ? (s % 8) ^ swz8(r) : (s % CH) ^ swz(r);
    const int rr = min(r, ti.nrows - 1);
    if (a_plane) {
      const int ar = sg.amap ? sg.amap[ti.row0 + rr] : ti.row0 + rr;
      a_off[j] = (uint32_t)(ar * APW + c * 8) * 2u;
    } else {
      const int ar = sg.amap ? sg.amap[ti.row0 + rr] : rr;
      a_off[j] = (uint32_t)(ar * K + c * 8) * 2u;
    }
  }
  // B: SwiGLU tiles take each wave column's RW rows as RW/2 rows of W1 then
  // the same columns of W3 (one descriptor each); the 64 slots of one load
  // are 64/CH consecutive rows inside one half, so the choice is uniform per
  // load.
  // K-blocked weights: the descriptor starts at the tile's first row in plane
  // 0 and spans the rest of the matrix; a lane's offset is its row's piece
  // in plane 0 and a stage adds its plane (one contiguous run per load).
  const int b_rows = (EPI == EPI_SWIGLU) ? BN / 2 : min(BN, sg.N - ncol0);
  const int b_plane = sg.b_blk ? sg.N * BK * M::WB : 0;
  const int b_step = sg.b_blk ? b_plane : BK * M::WB;  // bytes from one stage's slice to the next
  const size_t b_start = (size_t)ncol0 * (sg.b_blk ? BK : K) * M::WB;
  const int b_bytes = sg.b_blk ? (K / BK) * b_plane - ncol0 * BK * M::WB : b_rows * K * M::WB;
  const __amdgpu_buffer_rsrc_t b0_rsrc = uniform_rsrc(sg.B0 + b_start, b_bytes);
  const __amdgpu_buffer_rsrc_t b1_rsrc = uniform_rsrc((EPI == EPI_SWIGLU ? sg.B1 : sg.B0) + b_start, b_bytes);
  constexpr int BCH = BK * M::WB / 16;  // 16-byte chunks per weight row
  uint32_t b_off[M::B_LOADS];
  bool b_w3[M::B_LOADS];
#pragma unroll
  for (int j = 0; j < M::B_LOADS; ++j) {
    const int s = (wave * M::B_LOADS + j) * 64 + lane;
    const int r = s / BCH;
    const int c = (WDT == GD_FP8) ? ((s % BCH) ^ ((r >> 3) & 1)) : ((s % BCH) ^ swz(r));
    int n = r;  // row offset from ncol0
    b_w3[j] = false;
    if (EPI == EPI_SWIGLU) {
      const int half = C::RW / 2;
      const int r0 = (wave * M::B_LOADS + j) * 64 / BCH;
      b_w3[j] = (r0 % C::RW) >= half;
      n = (r / C::RW) * half + (r % C::RW) % half;
    }
    b_off[j] = (uint32_t)(n * (sg.b_blk ? BK : K) * M::WB + c * 16);
  }

  f32x4 acc[C::TW][C::TA];
#pragma unroll
  for (int i = 0; i < C::TW; ++i)
#pragma unroll
    for (int j = 0; j < C::TA; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A stage's fragments: the wave's weight blocks and activation blocks, 16
  // rows each.  Lane l takes row l % 16 of a block and the stage's k values
  // 8 (l / 16) .. 8 (l / 16) + 7: 16-byte chunk l / 16 of a bf16 row, bytes
  // 8 (l / 16) .. of a fp8 row (8 raw codes, widened to bf16 in registers).
  const int arow = wave_arow<BN, WN, LAY>(wave);
  const int kc = lane >> 4, rl = lane & 15;
  struct Frags {
    bf16x8 w[C::TW], x[C::TA];
  };
  u32x2 w8[C::TW];  // fp8: raw weight codes between their read and widening
  // A stage's LDS: its A (WIDE: the pair buffer and HALF, the stage's half
  // of each row) and its B.
  auto read_one = [&](Frags& F, const char* LA_, const char* LB_, auto HALF, auto POS) {
    constexpr int q = frag_order<C::TW, C::TA, WDT>(decltype(POS)::value);
    if constexpr (q < C::TW) {
      const int wr = wave_wrow<BN, WN, LAY, EPI, 16>(wave, q) + rl;
      if constexpr (WDT == GD_FP8)
        w8[q] = *(const u32x2*)(LB_ + f8_off(wr, kc >> 1) + (kc & 1) * 8);
      else
        F.w[q] = *(const bf16x8*)(LB_ + 2 * lds_off(wr, kc));
    } else {
      const int r = arow + (q - C::TW) * 16 + rl;
      if constexpr (WIDE)
        F.x[q - C::TW] = *(const bf16x8*)(LA_ + r * 128 + (((decltype(HALF)::value * 4 + kc) ^ swz8(r)) << 4));
      else
        F.x[q - C::TW] = *(const bf16x8*)(LA_ + 2 * lds_off(r, kc));
    }
  };
  auto widen = [&](Frags& F, auto I) {
    constexpr int i = decltype(I)::value;
    F.w[i] = e4m3x8_to_bf16(w8[i][0], w8[i][1]);
  };
  // WIDE: load l of the A refill of pair pp (stages 2 pp, 2 pp + 1 of the
  // piece; pairs past the end re-load the last one) into pair buffer pp % 2,
  // and load j of stage kt's B into B buffer kt % 4.
  auto issue_a2 = [&](int pp, auto LDX) {
    constexpr int l = decltype(LDX)::value;
    const int ps = kt0 / 2 + min(pp, KT / 2 - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        a_rsrc, (lds_ptr_t)(lds + (pp & 1) * A_PAIR + (wave * LA + l) * 1024), 16, a_off[l], ps * a_step, 0, 0);
  };
  auto issue_b2 = [&](int kt, auto JDX) {
    constexpr int j = decltype(JDX)::value;
    const int ks = kt0 + min(kt, KT - 1);
    const lds_ptr_t dst = (lds_ptr_t)(lds + 2 * A_PAIR + (kt & 3) * M::B_BYTES + (wave * M::B_LOADS + j) * 1024);
    if (b_w3[j])
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b1_rsrc, dst, 16, b_off[j], ks * b_step, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b0_rsrc, dst, 16, b_off[j], ks * b_step, 0, 0);
  };
  // load l of a stage: its A loads, then its B loads
  auto issue_one = [&](int kt, int buf, auto LDX) {
    constexpr int l = decltype(LDX)::value;
    char* st = lds + buf * M::STAGE_BYTES;
    const int ks = kt0 + min(kt, KT - 1);
    if constexpr (l < M::A_LOADS) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (lds_ptr_t)(st + (wave * M::A_LOADS + l) * 1024), 16, a_off[l], ks * a_step, 0, 0);
    } else if constexpr (l < M::LOADS) {
      constexpr int j = l - M::A_LOADS;
      const lds_ptr_t dst = (lds_ptr_t)(st + M::A_BYTES + (wave * M::B_LOADS + j) * 1024);
      if (b_w3[j])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b1_rsrc, dst, 16, b_off[j], ks * b_step, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b0_rsrc, dst, 16, b_off[j], ks * b_step, 0, 0);
    }
  };
  constexpr int NMF = C::TW * C::TA, NDS = C::TW + C::TA;  // MFMAs and fragment reads per stage
  auto mfma_range = [&](const Frags& F, auto LO, auto HI) {
    static_for<decltype(LO)::value, decltype(HI)::value>([&](auto MI) {
      constexpr int m = decltype(MI)::value;
      constexpr int i = m / C::TA, j = m % C::TA;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F.w[i], F.x[j], acc[i][j], 0, 0, 0);
    });
  };

  // Pipeline over a ring of STAGES = 4 buffers, stage kt in buffer kt % 4,
  // its fragments read into registers during stage kt - 1.  Stage kt is one
  // k32 step of TW x TA MFMAs on those registers, laid out as kNG groups
  // fenced so the compiler keeps the order:
  //   groups 0 .. kGB-1: MFMAs only;
  //   then every wave's reads of stage kt are done (lgkmcnt(0)) and this
  //     wave's loads of stage kt+1 have landed (vmcnt), and a barrier: stage
  //     kt+1 is readable and buffer kt % 4 free;
  //   groups kGB .. kNG-1: MFMAs, one direct load of stage kt+4 into buffer
  //     kt % 4 and a share of the reads of stage kt+1's fragments (fp8
  //     weights: raw codes, widened in the last groups).
  // A stage's loads are issued three stages before the barrier that waits
  // for them.  Stages past the end re-load the last k-slice into buffers
  // never read again, so every wait is a constant.
  //   WIDE: a pair buffer frees at the barrier of the pair's odd stage, so
  //     odd stage kt refills it with the A of stages kt+3 and kt+4 (two and
  //     three stages of lead); every stage refills its B buffer with stage
  //     kt+4's B.  The waits follow from that order.
  static_assert(STAGES == 4, "pipeline is laid out for 4 stages");
  static_assert(M::LOADS <= kNG - kGB && 3 * M::LOADS < 64, "loads per stage");
  static_assert(!WIDE || (LA + M::B_LOADS <= kNG - kGB && LA + 3 * M::B_LOADS < 64), "wide loads per stage");

  const bool scaled = WDT == GD_FP8 && EPI != EPI_BIAS_F32 && sg.s0 != nullptr && wk.slot < 0;
  if (scaled) stage_scales<BN, EPI, C::NTHR>(sg, ncol0, lds_sc, wave);
  if constexpr (WIDE) {
    static_for<0, LA>([&](auto J) { issue_a2(0, J); });
    static_for<0, M::B_LOADS>([&](auto J) { issue_b2(0, J); });
    static_for<0, M::B_LOADS>([&](auto J) { issue_b2(1, J); });
    static_for<0, LA>([&](auto J) { issue_a2(1, J); });
    static_for<0, M::B_LOADS>([&](auto J) { issue_b2(2, J); });
    static_for<0, M::B_LOADS>([&](auto J) { issue_b2(3, J); });
    wait_vmcnt<LA + 3 * M::B_LOADS>();  // stage 0 (and the scales) landed
  } else {
    static_for<0, STAGES>([&](auto S) {
      static_for<0, M::LOADS>([&](auto J) { issue_one(decltype(S)::value, decltype(S)::value, J); });
    });
    wait_vmcnt<3 * M::LOADS>();  // stage 0 (and the scales) landed
  }
  barrier_only();

  // stage u's LDS (u = kt % 4: every address a constant)
  auto a_lds = [&](auto U) -> const char* {
    constexpr int u = decltype(U)::value;
    return WIDE ? lds + ((u >> 1) & 1) * A_PAIR : lds + u * M::STAGE_BYTES;
  };
  auto b_lds = [&](auto U) -> const char* {
    constexpr int u = decltype(U)::value;
    return WIDE ? lds + 2 * A_PAIR + u * M::B_BYTES : lds + u * M::STAGE_BYTES + M::A_BYTES;
  };
  Frags F[2];
  static_for<0, NDS>([&](auto R) { read_one(F[0], a_lds(IC<0>{}), b_lds(IC<0>{}), IC<0>{}, R); });
  if constexpr (WDT == GD_FP8) static_for<0, C::TW>([&](auto I) { widen(F[0], I); });
  // unrolled by the ring depth: stage kt = k4 + u sits in buffer u, so
  // every LDS address is a constant
  for (int k4 = 0; k4 < KT; k4 += STAGES) {
    static_for<0, STAGES>([&](auto U) {
      constexpr int u = decltype(U)::value, cur = u & 1, un = (u + 1) % STAGES;
      const int kt = k4 + u;
      if (kt >= KT) return;
      const char* LAn = a_lds(IC<un>{});
      const char* LBn = b_lds(IC<un>{});
      // WIDE: loads after this stage's barrier (odd stages also refill A)
      constexpr int NL = WIDE ? ((u & 1) ? LA : 0) + M::B_LOADS : M::LOADS;
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, kGB>([&](auto G) {
        constexpr int g = decltype(G)::value;
        mfma_range(F[cur], IC<g * NMF / kNG>{}, IC<(g + 1) * NMF / kNG>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      if constexpr (!WIDE)
        wait_vmcnt<2 * M::LOADS>();
      else if constexpr (u & 1)
        wait_vmcnt<2 * M::B_LOADS>();
      else
        wait_vmcnt<LA + 2 * M::B_LOADS>();
      barrier_only();
      __builtin_amdgcn_sched_barrier(0);
      static_for<kGB, kNG>([&](auto G) {
        constexpr int g = decltype(G)::value, l = g - kGB;
        mfma_range(F[cur], IC<g * NMF / kNG>{}, IC<(g + 1) * NMF / kNG>{});
        if constexpr (!WIDE) {
          issue_one(kt + 4, u, IC<l>{});
        } else if constexpr (l < NL) {
          if constexpr ((u & 1) && l < LA)
            issue_a2((kt + 3) / 2, IC<l>{});
          else
            issue_b2(kt + 4, IC<l - ((u & 1) ? LA : 0)>{});
        }
        static_for<read_pos<NDS>(g), read_pos<NDS>(g + 1)>([&](auto R) {
          read_one(F[cur ^ 1], LAn, LBn, IC<un & 1>{}, R);
        });
        if constexpr (WDT == GD_FP8)
          static_for<0, C::TW>([&](auto I) {
            if constexpr (widen_group<C::TW, C::TA, WDT>(decltype(I)::value) == g) widen(F[cur ^ 1], I);
          });
        __builtin_amdgcn_sched_barrier(0);
      });
      if constexpr (WDT == GD_FP8)
        static_for<0, C::TW>([&](auto I) {
          if constexpr (widen_group<C::TW, C::TA, WDT>(decltype(I)::value) >= kNG) widen(F[cur ^ 1], I);
        });
    });
  }
  wait_vmcnt<0>();  // the re-loads past the end land before the block can exit

  if constexpr (EPI == EPI_BIAS_F32)  // router logits: never split (K ranges go to blockIdx.y)
    store_tile<C::TW, C::TA, WDT, EPI, 16>(a, ti, sg, acc, arow, ncol0 + wave_col<BN, WN, LAY, EPI>(wave), lane);
  else
    finish_tile<BN, WN, EPI, LAY, WDT, 16>(a, ti, sg, acc, ncol0, lds, wk.slot, lds_sc);
}
#endif

template <int BN, int WN, int EPI, int WDT>
__global__ __launch_bounds__(128 * WN, 1) void gemm_big_kernel(GemmArgs a, int n_tiles, int kt_plan,
                                                                int n_cu) {
  // device pass only: the host pass needs just the launch stub
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RING = STAGES * BigMem<BN, WN, 0, WDT>::STAGE_BYTES;
  constexpr int OUT = (EPI == EPI_BIAS_F32) ? 0 : OutTile<BN, EPI>::BYTES;
  constexpr int MAIN = RING > OUT ? RING : OUT;
  constexpr int SC = (WDT == GD_FP8 && EPI != EPI_BIAS_F32) ? BN * 4 : 0;  // the tile's channel scales
  __shared__ __attribute__((aligned(1024))) char lds[MAIN + SC];
  float* lds_sc = (float*)(lds + MAIN);
  Work wk;
  TileInfo ti;
  Seg sg;
  constexpr int NCOLS = EPI == EPI_SWIGLU ? BN / 2 : BN;
  if (!big_block(a, n_tiles, kt_plan, n_cu, m_tile_rows(a), NCOLS, wk, ti, sg)) return;
  const int ncol0 = wk.nt * NCOLS;
  if constexpr (EPI == EPI_SWIGLU) {
    if (sg.a_wide) {  // A in 64-column planes (checked by the launcher: K % 64 == 0)
      switch (tile_layout(ti.nrows)) {
        case 2: big_tile<BN, WN, EPI, 2, WDT, true>(a, ti, sg, wk, ncol0, lds, lds_sc); break;
        case 1: big_tile<BN, WN, EPI, 1, WDT, true>(a, ti, sg, wk, ncol0, lds, lds_sc); break;
        default: big_tile<BN, WN, EPI, 0, WDT, true>(a, ti, sg, wk, ncol0, lds, lds_sc);
      }
      return;
    }
  }
  switch (tile_layout(ti.nrows)) {
    case 2: big_tile<BN, WN, EPI, 2, WDT, false>(a, ti, sg, wk, ncol0, lds, lds_sc); break;
    case 1: big_tile<BN, WN, EPI, 1, WDT, false>(a, ti, sg, wk, ncol0, lds, lds_sc); break;
    default: big_tile<BN, WN, EPI, 0, WDT, false>(a, ti, sg, wk, ncol0, lds, lds_sc);
  }
#endif
}


// ---------------------------------------------------------------------------
// fp8 x fp8 gate-up tiles: activations are the block-scaled E4M3 dispatch
// payload (codes, and one E8M0 scale per 32 k values of a row), weights are
// E4M3 with per-output-channel fp32 scales.  v_mfma_scale_f32_32x32x64_f8f6f4
// takes, per lane, 32 k values of one row of each operand (two 16-value
// halves, one from each 32-value block, measured on gfx950) and one E8M0
// scale per lane: lane half h's scale multiplies k-block h.  The activation
// scale is that block's payload scale, the weight scale 2^0 (the channel
// scales are applied in the epilogue as on the bf16 path).
// Per k, an fp8 MFMA takes half the cycles and each operand half the bytes
// of bf16, so a stage holds BK8 = 64 k values in the same 64-byte LDS rows
// and the same ring of four 32 KB stages.  The activation scales come in
// 16-byte chunks per row (16 blocks, 8 stages) through a two-slot LDS ring
// refilled once per 8 stages; K-pieces of split tiles start on chunk
// boundaries.
//
// A stage (k = 64) is one step of TW x TA block-scaled MFMAs, laid out like
// a stage of the bf16 pipeline: groups of MFMAs, each followed by its
// share of the direct loads and of the next stage's fragment reads (full
// fragment sets double-buffered in registers).  The first groups issue the B
// refill, then the barrier, then the A refill and the reads (Qwen-shaped
// fp8 x fp8 gate-up 918 -> 904 us against a schedule of four quarters with
// the loads issued four at a time).
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int BK8 = 64;            // k per stage of the fp8 x fp8 path
[[maybe_unused]] constexpr int SC_STAGES = 8;       // stages per 16-byte chunk of scales
[[maybe_unused]] constexpr int SC_BYTES = BM * 16;  // one chunk for every row of a tile

#if defined(__HIP_DEVICE_COMPILE__)
template <int BN, int WN, int EPI, int LAY>
__device__ __forceinline__ void big_tile_fp8(const GemmArgs& a, const TileInfo& ti, const Seg& sg, const Work& wk,
                                             int ncol0, char* lds, float* lds_sc) {
  using C = BigCfg<BN, WN, LAY>;
  using M = BigMem<BN, WN, LAY, GD_BF16>;  // 64-byte rows on both operands: the bf16 stage geometry
  static_assert(C::NTHR == BM, "one scale row per thread");
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = sg.K;  // bytes per row of either operand
  // this block's chunks of 8 stages: all, or piece k0num of s
  const int KT_all = K / BK8, NCK = (KT_all + SC_STAGES - 1) / SC_STAGES;
  const int ck0 = wk.k0num * NCK / wk.s, ck1 = (wk.k0num + 1) * NCK / wk.s;
  const int kt0 = ck0 * SC_STAGES, KT = min(ck1 * SC_STAGES, KT_all) - kt0, NC = ck1 - ck0;

  const __amdgpu_buffer_rsrc_t a_rsrc =
      sg.amap ? uniform_rsrc(sg.A, a.a_map_rows * K) : uniform_rsrc(sg.A + (size_t)ti.row0 * K, ti.nrows * K);
  uint32_t a_off[M::A_LOADS];
#pragma unroll
  for (int j = 0; j < M::A_LOADS; ++j) {
    const int s = (wave * M::A_LOADS + j) * 64 + lane;
    const int r = s / CH, c = (s % CH) ^ swz(r);
    const int rr = min(r, ti.nrows - 1);
    const int ar = sg.amap ? sg.amap[ti.row0 + rr] : rr;
    a_off[j] = (uint32_t)(ar * K + c * 16);
  }
  const int b_rows = (EPI == EPI_SWIGLU) ? BN / 2 : min(BN, sg.N - ncol0);
  // K-blocked weights: a 64-k stage spans two 32-column planes of N x 32 bytes
  const int b_plane = sg.b_blk ? sg.N * 32 : 0;
  const size_t b_start = (size_t)ncol0 * (sg.b_blk ? 32 : K);
  const int b_bytes = sg.b_blk ? (K / 32) * b_plane - ncol0 * 32 : b_rows * K;
  const __amdgpu_buffer_rsrc_t b0_rsrc = uniform_rsrc(sg.B0 + b_start, b_bytes);
  const __amdgpu_buffer_rsrc_t b1_rsrc = uniform_rsrc((EPI == EPI_SWIGLU ? sg.B1 : sg.B0) + b_start, b_bytes);
  const int b_step = sg.b_blk ? 2 * b_plane : BK8;
  uint32_t b_off[M::B_LOADS];
  bool b_w3[M::B_LOADS];
#pragma unroll
  for (int j = 0; j < M::B_LOADS; ++j) {
    const int s = (wave * M::B_LOADS + j) * 64 + lane;
    const int r = s / CH, c = (s % CH) ^ swz(r);
    int n = r;
    b_w3[j] = false;
    if (EPI == EPI_SWIGLU) {
      const int half = C::RW / 2;
      const int r0 = (wave * M::B_LOADS + j) * 64 / CH;
      b_w3[j] = (r0 % C::RW) >= half;
      n = (r / C::RW) * half + (r % C::RW) % half;
    }
    b_off[j] = sg.b_blk ? (uint32_t)((c >> 1) * b_plane + n * 32 + (c & 1) * 16) : (uint32_t)(n * K + c * 16);
  }
  // scales: thread t loads the chunk of tile row t (rows past the tile's
  // end repeat its last row); waves past the loaded rows load nothing
  const uint8_t* s_base = sg.amap ? a.a_scales : a.a_scales + (size_t)ti.row0 * a.a_sstride;
  const int s_rows = sg.amap ? a.a_map_rows : ti.nrows;
  const __amdgpu_buffer_rsrc_t s_rsrc = uniform_rsrc(s_base, s_rows * a.a_sstride);
  uint32_t s_off;
  {
    const int rr = min(tid, ti.nrows - 1);
    const int ar = sg.amap ? sg.amap[ti.row0 + rr] : rr;
    s_off = (uint32_t)(ar * a.a_sstride + ck0 * 16);
  }
  char* sring = lds + STAGES * M::STAGE_BYTES;

  auto issue_part = [&](int kt, int buf, int part) {
    char* st = lds + buf * M::STAGE_BYTES;
    const int ks = kt0 + min(kt, KT - 1);
    if (part == 0) {
#pragma unroll
      for (int j = 0; j < M::A_LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (lds_ptr_t)(st + (wave * M::A_LOADS + j) * 1024), 16, a_off[j], ks * BK8, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < M::B_LOADS; ++j) {
        const lds_ptr_t dst = (lds_ptr_t)(st + M::A_BYTES + (wave * M::B_LOADS + j) * 1024);
        if (b_w3[j])
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b1_rsrc, dst, 16, b_off[j], ks * b_step, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b0_rsrc, dst, 16, b_off[j], ks * b_step, 0, 0);
      }
    }
  };
  auto issue_scales = [&](int c) {  // piece chunk c (clamped) into ring slot c & 1
    if (wave * 64 < C::A_ROWS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr_t)(sring + (c & 1) * SC_BYTES + wave * 1024), 16,
                                               s_off, min(c, NC - 1) * 16, 0, 0);
  };

  f32x16 acc[C::TW][C::TA];
#pragma unroll
  for (int i = 0; i < C::TW; ++i)
#pragma unroll
    for (int j = 0; j < C::TA; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int arow = wave_arow<BN, WN, LAY>(wave);
  // The lane's 32 bytes of an LDS row: the MFMA takes k values 16h..16h+15
  // from bytes 0-15 and 32+16h..32+16h+15 from bytes 16-31 of lane half h
  // (16-byte chunks h and h + 2 of the 64-k row), and lane half h's scale
  // covers k-block h (k 32h..32h+31).
  auto frag = [&](const char* base, int r) -> i32x8 {
    const i32x4 p = *(const i32x4*)(base + 2 * lds_off(r, h));
    const i32x4 q = *(const i32x4*)(base + 2 * lds_off(r, h + 2));
    return __builtin_shufflevector(p, q, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto wfrag = [&](const char* L, int i) {
    return frag(L + M::A_BYTES, wave_wrow<BN, WN, LAY, EPI, 32>(wave, i) + (lane & 31));
  };
  auto xfrag = [&](const char* L, int j) { return frag(L, arow + j * 32 + (lane & 31)); };
  u32x4 SC[C::TA];  // this chunk's 16 scale bytes of each activation block's row
  auto read_scales = [&](int c) {
#pragma unroll
    for (int j = 0; j < C::TA; ++j)
      SC[j] = *(const u32x4*)(sring + (c & 1) * SC_BYTES + (arow + j * 32 + (lane & 31)) * 16);
  };
  auto mf = [&](int i, int j, const i32x8& w, const i32x8& x, int sb) {
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, acc[i][j], 0, 0, 0, 127, 0, sb);
  };

  // Fragments of one stage (k = 64): the wave's weight and activation
  // blocks, 32 bytes of a row per lane.  F[st & 1] holds stage st's.
  struct Frags8 {
    i32x8 w[C::TW], x[C::TA];
  };
  constexpr int NMF = C::TW * C::TA, NDS = C::TW + C::TA;  // MFMAs and fragments per stage
  constexpr int NG = NDS;                                  // groups per stage
  constexpr int BG = 2;                                    // groups before the barrier
  static_assert(BG >= 1 && BG < NG, "barrier group");
  // fragment q of a stage in the order the MFMAs (i-major) consume them:
  // w0, every x, then w1 ..
  auto read_one = [&](Frags8& F, const char* L, auto IDX) {
    constexpr int qq = decltype(IDX)::value;
    constexpr int q = qq == 0 ? 0 : qq <= C::TA ? C::TW + qq - 1 : qq - C::TA;
    if constexpr (q < C::TW) F.w[q] = wfrag(L, q);
    else F.x[q - C::TW] = xfrag(L, q - C::TW);
  };
  auto load_one = [&](int kt, int buf, int part, auto JDX) {
    constexpr int jj = decltype(JDX)::value;
    char* st = lds + buf * M::STAGE_BYTES;
    const int ks = kt0 + min(kt, KT - 1);
    if (part == 0) {
      if constexpr (jj < M::A_LOADS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (lds_ptr_t)(st + (wave * M::A_LOADS + jj) * 1024), 16, a_off[jj], ks * BK8, 0, 0);
    } else {
      if constexpr (jj < M::B_LOADS) {
        const lds_ptr_t dst = (lds_ptr_t)(st + M::A_BYTES + (wave * M::B_LOADS + jj) * 1024);
        if (b_w3[jj])
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b1_rsrc, dst, 16, b_off[jj], ks * b_step, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b0_rsrc, dst, 16, b_off[jj], ks * b_step, 0, 0);
      }
    }
  };
  auto mfma_range = [&](const Frags8& F, const int (&sb)[C::TA], auto LO, auto HI) {
    static_for<decltype(LO)::value, decltype(HI)::value>([&](auto MI) {
      constexpr int m = decltype(MI)::value;
      constexpr int i = m / C::TA, j = m % C::TA;
      mf(i, j, F.w[i], F.x[j], sb[j]);
    });
  };

  // prologue: the channel scales, scale chunk 0, stages 0..2 and the A part
  // of stage 3
  const bool scaled = sg.s0 != nullptr && wk.slot < 0;
  if (scaled) stage_scales<BN, EPI, C::NTHR>(sg, ncol0, lds_sc, wave);
  issue_scales(0);
  issue_part(0, 0, 0); issue_part(0, 0, 1);
  issue_part(1, 1, 0); issue_part(1, 1, 1);
  issue_part(2, 2, 0); issue_part(2, 2, 1);
  issue_part(3, 3, 0);
  wait_vmcnt<2 * M::LOADS + M::A_LOADS>();  // scale chunk 0 and stage 0 done
  barrier_only();
  read_scales(0);
  Frags8 F[2];
  static_for<0, NDS>([&](auto Q) { read_one(F[0], lds, Q); });

  // Stage kt is in ring buffer kt % 4 = st % 4 (chunks are 8 stages), so
  // every LDS address is a constant.  A stage is laid out as NG groups, each
  // fenced so the compiler keeps the order: a group's MFMAs on F[st & 1],
  // then its share of the direct loads and of the next stage's fragment
  // reads.  The first BG groups issue the B part of stage kt+3 (into buffer
  // (kt+3) % 4, whose stage every wave had read before the previous barrier);
  // then this wave's loads of stage kt+1 have landed and a barrier (every wave
  // holds this stage's fragments, so buffer kt % 4 is free); the remaining
  // groups issue the A part of stage kt+4 into buffer kt % 4 and read stage
  // kt+1's fragments into F[(st + 1) & 1].  Waits are those of the bf16
  // pipeline; a scale chunk load adds one more load to some waits' windows,
  // which only makes them wait a little longer.
  for (int c = 0; c < NC; ++c) {
    static_for<0, SC_STAGES>([&](auto ST) {
      constexpr int st = decltype(ST)::value, p = st & 1;
      const int kt = c * SC_STAGES + st;
      if (kt >= KT) return;
      const char* Ln = lds + ((st + 1) % STAGES) * M::STAGE_BYTES;
      constexpr int bb = (st + 3) % STAGES, ba = st % STAGES;
      int sb[C::TA];
#pragma unroll
      for (int j = 0; j < C::TA; ++j) sb[j] = (int)((SC[j][st >> 1] >> (16 * (st & 1) + 8 * h)) & 0xffu);
      if (st == 0) issue_scales(c + 1);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, BG>([&](auto G) {
        constexpr int g = decltype(G)::value;
        mfma_range(F[p], sb, IC<g * NMF / NG>{}, IC<(g + 1) * NMF / NG>{});
        static_for<g * M::B_LOADS / BG, (g + 1) * M::B_LOADS / BG>([&](auto J) { load_one(kt + 3, bb, 1, J); });
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      wait_vmcnt<2 * M::LOADS>();
      barrier_only();
      __builtin_amdgcn_sched_barrier(0);
      static_for<BG, NG>([&](auto G) {
        constexpr int g = decltype(G)::value, q0 = g - BG, NP = NG - BG;
        mfma_range(F[p], sb, IC<g * NMF / NG>{}, IC<(g + 1) * NMF / NG>{});
        static_for<q0 * M::A_LOADS / NP, (q0 + 1) * M::A_LOADS / NP>([&](auto J) { load_one(kt + 4, ba, 0, J); });
        static_for<q0 * NDS / NP, (q0 + 1) * NDS / NP>([&](auto R) { read_one(F[p ^ 1], Ln, R); });
        if constexpr (g == NG - 1 && st == SC_STAGES - 1) read_scales(c + 1);
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  }
  wait_vmcnt<0>();  // the re-loads past the end land before the block can exit
  finish_tile<BN, WN, EPI, LAY, GD_FP8, 32>(a, ti, sg, acc, ncol0, lds, wk.slot, lds_sc);
}
#endif

template <int BN, int WN, int EPI>
__global__ __launch_bounds__(128 * WN, 1) void gemm_big_fp8_kernel(GemmArgs a, int n_tiles, int kt_plan,
                                                                    int n_cu) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(OutTile<BN, EPI>::BYTES <= STAGES * BigMem<BN, WN, 0, GD_BF16>::STAGE_BYTES, "LDS");
  constexpr int MAIN = STAGES * BigMem<BN, WN, 0, GD_BF16>::STAGE_BYTES + 2 * SC_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[MAIN + BN * 4];  // + the tile's channel scales
  float* lds_sc = (float*)(lds + MAIN);
  Work wk;
  TileInfo ti;
  Seg sg;
  constexpr int NCOLS = EPI == EPI_SWIGLU ? BN / 2 : BN;
  if (!big_block(a, n_tiles, kt_plan, n_cu, BM, NCOLS, wk, ti, sg)) return;
  const int ncol0 = wk.nt * NCOLS;
  switch (tile_layout(ti.nrows)) {
    case 2: big_tile_fp8<BN, WN, EPI, 2>(a, ti, sg, wk, ncol0, lds, lds_sc); break;
    case 1: big_tile_fp8<BN, WN, EPI, 1>(a, ti, sg, wk, ncol0, lds, lds_sc); break;
    default: big_tile_fp8<BN, WN, EPI, 0>(a, ti, sg, wk, ncol0, lds, lds_sc);
  }
#endif
}

// Fixup of the split tiles, one float4 of the pieces' register layout per
// work unit: unit ((i * TA + j) * RUNS + g) * NTHR + t holds accumulator
// floats 4g..4g+3 of block (i, j) of GEMM thread t, i.e. four consecutive
// output columns of one row (the block layout of finish_tile, edge BH).  The unit's pieces are added in piece order (the same
// sum whichever block ran which piece), then the tile's epilogue is applied
// to those four columns.  SwiGLU units pair block i (u) with block i + TW/2
// (v).  Spreading units over many blocks keeps the reads in flight.
constexpr int kFixupChunks = 16;  // blocks per split tile
template <int BN, int WN, int EPI, int LAY, int WDT, int BH>
__device__ __forceinline__ void fixup_units(const GemmArgs& a, const TileInfo& ti, const Seg& sg, int ncol0,
                                            int first_slot, int s) {
  using C = BigCfg<BN, WN, LAY, BH>;
  constexpr int NT = 128 * WN;  // threads of the GEMM block
  constexpr int TWO = (EPI == EPI_SWIGLU) ? C::TW / 2 : C::TW;
  constexpr int UNITS = NT * TWO * C::TA * C::RUNS;
  constexpr size_t SLOT4 = kPartialSlotBytes / 16;
  const float4* P = (const float4*)a.partial + (size_t)first_slot * SLOT4;
  // pieces in order; their loads four at a time, so several are in flight
  auto sum = [&](int e) {
    float4 x = P[e];
    auto add = [&](const float4& y) {
      x.x += y.x;
      x.y += y.y;
      x.z += y.z;
      x.w += y.w;
    };
    int p = 1;
    for (; p + 4 <= s; p += 4) {
      float4 y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = P[(size_t)(p + q) * SLOT4 + e];
#pragma unroll
      for (int q = 0; q < 4; ++q) add(y[q]);
    }
    for (; p < s; ++p) add(P[(size_t)p * SLOT4 + e]);
    return x;
  };
  for (int u = blockIdx.y * blockDim.x + threadIdx.x; u < UNITS; u += gridDim.y * blockDim.x) {
    const int t = u % NT, r = u / NT;
    const int g = r % C::RUNS, j = (r / C::RUNS) % C::TA, i = (r / C::RUNS) / C::TA;
    const int wave = t >> 6, lane = t & 63;
    const int row = wave_arow<BN, WN, LAY>(wave) + j * BH + lane % BH;
    if (row >= ti.nrows) continue;
    const int n = ncol0 + wave_col<BN, WN, LAY, EPI>(wave) + i * BH + g * 8 + (lane / BH) * 4;
    float o[4];
    const float4 x = sum(((i * C::TA + j) * C::RUNS + g) * NT + t);
    if (EPI == EPI_SWIGLU) {
      const float4 y = sum((((i + C::TW / 2) * C::TA + j) * C::RUNS + g) * NT + t);
      float4 su = make_float4(1.f, 1.f, 1.f, 1.f), sv = su;
      if (WDT == GD_FP8 && sg.s0) {
        su = *(const float4*)(sg.s0 + n);
        sv = *(const float4*)(sg.s1 + n);
      }
      o[0] = silu(x.x * su.x) * (y.x * sv.x);
      o[1] = silu(x.y * su.y) * (y.y * sv.y);
      o[2] = silu(x.z * su.z) * (y.z * sv.z);
      o[3] = silu(x.w * su.w) * (y.w * sv.w);
    } else {
      float4 sc = make_float4(1.f, 1.f, 1.f, 1.f);
      if (WDT == GD_FP8 && sg.s0) sc = *(const float4*)(sg.s0 + n);
      o[0] = x.x * sc.x;
      o[1] = x.y * sc.y;
      o[2] = x.z * sc.z;
      o[3] = x.w * sc.w;
    }
    u32x2 v;
    v[0] = pack_bf16x2(o[0], o[1]);
    v[1] = pack_bf16x2(o[2], o[3]);
    // n is a multiple of 4: the four columns lie in one 32-column plane
    const size_t at = sg.c_prows ? ((size_t)(n / 32) * sg.c_prows + ti.row0 + row) * 32 + n % 32
                                 : (size_t)(ti.row0 + row) * sg.N + n;
    *(u32x2*)((uint16_t*)sg.C + at) = v;
  }
}

// Blocks (split tile, chunk); BH: the MFMA block edge of the GEMM's tiles.
template <int BN, int WN, int EPI, int WDT, int BH>
__global__ __launch_bounds__(256) void gemm_big_fixup_kernel(GemmArgs a, int n_tiles, int kt_plan, int n_cu) {
  if constexpr (EPI != EPI_BIAS_F32) {  // router logits never split this way
    const int m_real = real_mtiles(a, BM);
    const SplitPlan p = split_plan(m_real * n_tiles, kt_plan, n_cu, a.partial ? a.partial_slots : 0);
    if ((int)blockIdx.x >= p.rem) return;
    int mt, nt;
    tile_coords(p.full + blockIdx.x, m_real, n_tiles, mt, nt);
    TileInfo ti;
    Seg sg;
    if (!tile_info(a, mt, BM, ti, sg)) return;
    const int ncol0 = nt * (EPI == EPI_SWIGLU ? BN / 2 : BN);
    if (ncol0 >= sg.N) return;
    switch (tile_layout(ti.nrows)) {
      case 2: fixup_units<BN, WN, EPI, 2, WDT, BH>(a, ti, sg, ncol0, blockIdx.x * p.s, p.s); break;
      case 1: fixup_units<BN, WN, EPI, 1, WDT, BH>(a, ti, sg, ncol0, blockIdx.x * p.s, p.s); break;
      default: fixup_units<BN, WN, EPI, 0, WDT, BH>(a, ti, sg, ncol0, blockIdx.x * p.s, p.s);
    }
  }
}

// Compute units of the current device (the split plan fills one wave of them),
// cached per device.  Calls from several threads may race to fill an entry;
// each stores the same value, and the entries are atomic, so that is benign.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int BN, int EPI, int WDT, bool FP8ACT = false, int WN = MOE_BIG_WN>
hipError_t launch_big(const GemmArgs& a_in, hipStream_t s) {
  GemmArgs a = a_in;
  const int n_slots = a.tile_table ? a.n_slots : (a.rows + m_tile_rows(a) - 1) / m_tile_rows(a);
  const int ncol = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int n_tiles = (gemm_max_cols(a) + ncol - 1) / ncol;
  const int kt_plan = (a.sh_rows > 0 ? min(a.K, a.shK) : a.K) / (FP8ACT ? BK8 : BK);
  int n_cu = device_cus();
  if (a.ksplit < 1) a.ksplit = 1;
  if (n_cu <= 0 || n_cu % 8 != 0 || a.partial == nullptr || a.ksplit > 1) {
    n_cu = 0;  // no split: every tile runs whole
    a.partial = nullptr;
    a.partial_slots = 0;
  }
  a.partial_slots = min(a.partial_slots, kPartialSlots);
  // whole tiles plus at most one wave of pieces, 8 XCD shares rounded up
  int nb = n_slots * n_tiles + (n_cu > 0 ? n_cu + 8 : 0);
  nb = (nb + 7) & ~7;
  // Each block's tile resolved ahead by one thread per block (the tile
  // table's real m-tile count, the grouped order and split plan, the table
  // entry and the segment's offsets), so a GEMM block starts from one record
  // instead of a chain of dependent loads and divisions.
  if (a.sched != nullptr && a.tile_table != nullptr && a.ksplit == 1 && nb <= a.sched_cap)
    hipLaunchKernelGGL(big_sched_kernel, dim3((nb + 255) / 256), dim3(256), 0, s, a, n_tiles, kt_plan, n_cu, BM,
                       ncol, nb);
  else
    a.sched = nullptr;
  if constexpr (FP8ACT)
    hipLaunchKernelGGL((gemm_big_fp8_kernel<BN, WN, EPI>), dim3(nb), dim3(128 * WN), 0, s, a, n_tiles, kt_plan,
                       n_cu);
  else
    hipLaunchKernelGGL((gemm_big_kernel<BN, WN, EPI, WDT>), dim3(nb, a.ksplit), dim3(128 * WN), 0, s, a,
                       n_tiles, kt_plan, n_cu);
  if (n_cu > 0)
    hipLaunchKernelGGL((gemm_big_fixup_kernel<BN, WN, EPI, WDT, FP8ACT ? 32 : 16>), dim3(n_cu / 2, kFixupChunks), dim3(256),
                       0, s, a, n_tiles, kt_plan, n_cu);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_big(const GemmArgs& a, hipStream_t s) {
  if (a.act == GD_FP8) return launch_big<256, EPI_SWIGLU, GD_FP8, true>(a, s);  // checked by the caller
  if (a.epi == EPI_BIAS_F32)  // router logits: 128-wide tiles unless E fills 256-wide ones
    return (a.N % 256 == 0) ? launch_big<256, EPI_BIAS_F32, GD_BF16>(a, s) : launch_big<128, EPI_BIAS_F32, GD_BF16>(a, s);
  if (a.wdt == GD_FP8) {
    if (a.epi == EPI_SWIGLU) return launch_big<256, EPI_SWIGLU, GD_FP8>(a, s);
    return (a.N % 256 == 0) ? launch_big<256, EPI_STORE, GD_FP8>(a, s) : launch_big<128, EPI_STORE, GD_FP8>(a, s);
  }
  if (a.epi == EPI_SWIGLU) return launch_big<256, EPI_SWIGLU, GD_BF16>(a, s);
  return (a.N % 256 == 0) ? launch_big<256, EPI_STORE, GD_BF16>(a, s) : launch_big<128, EPI_STORE, GD_BF16>(a, s);
}

}  // namespace moe
