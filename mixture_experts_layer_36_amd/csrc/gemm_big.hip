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
//     128 x (BN/2) tile: 16 (or 8) v_mfma_f32_32x32x16_bf16 per 8 (or 6)
//     128-bit LDS fragment reads, with the accumulators in AGPRs;
//   * global -> LDS with global_load_lds_dwordx4 (no VGPR staging) into a
//     4-deep ring of 32 KB stages, refilled four stages ahead; each wave
//     waits only for its own loads of the next stage (vmcnt) and a bare
//     s_barrier publishes them, so later stages stay in flight;
//   * the LDS fragments of the next k16 step are read while the current
//     step's MFMAs run (two fragment sets, interleaved by
//     sched_group_barrier), across the stage boundary too;
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
//     ((r >> 2) & 3 for 64-byte rows, (r ^ (r >> 3)) & 7 for 128-byte rows):
//     measured on gfx950 (64 banks; a 128-bit read is served 16 lanes at a
//     time), these make the fragment reads of 32 rows x 1 chunk
//     conflict-free.  A direct load writes 64 consecutive 16-byte slots, so
//     each lane fetches the global chunk that belongs in its slot;
//   * operands row-major or K-blocked (32-column planes of [rows][32]: the
//     expert weights when packed, h between the two routed GEMMs, x_perm for
//     wide experts): K-blocked, a stage's slice of a tile's consecutive rows
//     is one contiguous run, so a 1 KB direct load covers 8 whole cache
//     lines instead of 16 half lines;
//   * every buffer descriptor is built from block-uniform values stated
//     uniform (readfirstlane): otherwise the compiler cannot prove a base
//     computed on the vector unit uniform and wraps each load through it in a
//     loop over distinct lane values.
#include <atomic>

#include "gemm_common.hpp"

namespace moe {
namespace {

#ifndef MOE_BIG_WN
#define MOE_BIG_WN 2
#endif
constexpr int BM = 256, BK = 32, STAGES = 4;
constexpr int CH = BK / 8;        // 16-byte chunks per LDS row
[[maybe_unused]] constexpr int KK = BK / 16;       // k16 MFMA steps per stage

// Tile layouts, LAY = 0, 1, 2.  Full (0): WN wavefronts along the weight
// rows, 2 along the 256 activation rows, each wave 128 activation rows x RW
// weight rows.  Half (1, tiles of at most 128 rows): all 2*WN wavefronts on
// the 128 activation rows, each with RW/2 weight rows.  Quarter (2, at most
// 64 rows): the same weight split over 64 activation rows.  The LDS ring is
// the same; a shorter layout loads and multiplies only its rows.
template <int BN, int WN, int LAY>
struct BigCfg {
  static constexpr int NTHR = 128 * WN;
  static constexpr int RW = BN / WN;                 // weight rows per wave column (full layout)
  static constexpr int TA = LAY == 2 ? 2 : 4;        // 32-row activation blocks per wave
  static constexpr int TW = LAY ? RW / 64 : RW / 32;
  static constexpr int A_ROWS = BM >> LAY;           // activation rows loaded
  static_assert(TW >= 1 && LAY >= 0 && LAY <= 2, "layout");
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
// value): the hardware conversion to f32, then the upper halves.
[[maybe_unused]] __device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4 o;
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  o[0] = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
  o[1] = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
  o[2] = __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), 0x07060302u);
  o[3] = __builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), 0x07060302u);
  return __builtin_bit_cast(bf16x8, o);
}

// LDS weight row of a wave's block i, its first activation row and the first
// output column of its blocks (relative to the tile's first column).  SwiGLU
// tiles hold, per wave column of the full layout, RW/2 rows of W1 followed
// by the same columns of W3, and a wave's blocks i < TW/2 are W1 (u), the
// blocks i + TW/2 the matching W3 (v).
template <int BN, int WN, int LAY, int EPI>
__device__ __forceinline__ int wave_wrow(int wave, int i) {
  using C = BigCfg<BN, WN, LAY>;
  if (!LAY) return (wave % WN) * C::RW + i * 32;
  if (EPI != EPI_SWIGLU) return wave * (C::RW / 2) + i * 32;
  const int slab = wave >> 1, sub = wave & 1;
  return i < C::TW / 2 ? slab * C::RW + sub * (C::RW / 4) + i * 32
                       : slab * C::RW + C::RW / 2 + sub * (C::RW / 4) + (i - C::TW / 2) * 32;
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
// tiles come first, an equal contiguous share per XCD (grouped order, so the
// blocks an XCD runs at once share operands in its L2); the split pieces
// follow, again an equal share per XCD, so they all run in the last wave.
[[maybe_unused]] __device__ __forceinline__ bool big_work(const GemmArgs& a, int n_tiles, int kt_plan, int n_cu,
                                         int BMv, Work& w) {
  const int m_real = real_mtiles(a, BMv);
  const int R = m_real * n_tiles;
  const SplitPlan p = split_plan(R, kt_plan, n_cu, a.partial ? a.partial_slots : 0);
  const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
  int L;
  w.slot = -1;
  w.k0num = 0;
  w.s = 1;
  if (p.rem > 0) {
    const int f8 = p.full >> 3, Q = p.rem * p.s, q = (Q + 7) >> 3;
    if (i < f8) {
      L = x * f8 + i;
    } else {
      const int j = i - f8, pi = x * q + j;
      if (j >= q || pi >= Q) return false;
      L = p.full + pi / p.s;
      w.k0num = pi % p.s;
      w.slot = pi;
      w.s = p.s;
    }
  } else {
    const int share = (R + 7) >> 3;
    L = x * share + i;
    if (i >= share || L >= R) return false;
  }
  tile_coords(L, m_real, n_tiles, w.mt, w.nt);
  return true;
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
// K-piece of a split tile.
//   * A whole tile goes out through LDS: each wave writes its values -- runs
//     of 4 consecutive columns of one row per lane and 32x32 block -- into a
//     row-major copy of the tile, 16-byte chunk c of row r at c ^ (r & 15)
//     (the 32 rows one write touches spread over the banks); then the block
//     stores whole rows with 16-byte writes, so one wave instruction covers
//     2-4 full row runs rather than 32 rows x 16 bytes.  The operand ring is
//     dead by then: every wave has read its last fragments.
//   * A piece stores its raw accumulators to its partial slot, register-major
//     so that each 16-byte store of a wave is contiguous.
// Both are handled block by block in one pass.
template <int BN, int WN, int EPI, int LAY, int WDT>
__device__ __forceinline__ void finish_tile(const GemmArgs& a, const TileInfo& ti, const Seg& sg,
                                            f32x16 (&acc)[BigCfg<BN, WN, LAY>::TW][BigCfg<BN, WN, LAY>::TA],
                                            int ncol0, char* lds, int slot) {
  using C = BigCfg<BN, WN, LAY>;
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
    P[((i * C::TA + j) * 4 + g) * C::NTHR + tid] =
        make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
  };
  constexpr int NB = (EPI == EPI_SWIGLU) ? C::TW / 2 : C::TW;
#pragma unroll
  // Column group by column group (4 columns of 32 activation rows per lane
  // and block): only that group's fp8 channel scales stay live, which cuts
  // the fp8-weight epilogue's register spills by more than half.
  for (int i = 0; i < NB; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int lcol = wcol + i * 32 + g * 8 + (lane >> 5) * 4;
      float4 su = make_float4(1.f, 1.f, 1.f, 1.f), sv = su;
      if (scaled) {
        su = *(const float4*)(sg.s0 + ncol0 + lcol);
        if (EPI == EPI_SWIGLU) sv = *(const float4*)(sg.s1 + ncol0 + lcol);
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
        const int lrow = arow + j * 32 + (lane & 31);
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
      // one group at a time: the accumulators leave the AGPRs as needed
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (piece) return;
  __builtin_amdgcn_s_waitcnt(0xc07f);
  barrier_only();
  const int rows = ti.nrows;
  if (sg.c_prows) {
    // K-blocked C: the tile's 32-column planes in turn, each a contiguous run
    // of rows x 64 bytes (4 chunks per row)
    for (int u = tid; u < rows * O::CPR; u += C::NTHR) {
      const int p = u / (rows * 4), rem = u % (rows * 4), r = rem >> 2, ch = p * 4 + (rem & 3);
      const u32x4 v = *(const u32x4*)(lds + r * O::ROW_BYTES + ((ch ^ (r & 15)) << 4));
      if (ncol0 + p * 32 < sg.N)
        *(u32x4*)((uint16_t*)sg.C + ((size_t)(ncol0 / 32 + p) * sg.c_prows + ti.row0 + r) * 32 + (rem & 3) * 8) = v;
    }
    return;
  }
  for (int u = tid; u < rows * O::CPR; u += C::NTHR) {
    const int r = u / O::CPR, ch = u % O::CPR;
    const u32x4 v = *(const u32x4*)(lds + r * O::ROW_BYTES + ((ch ^ (r & 15)) << 4));
    if (ncol0 + ch * 8 < sg.N) *(u32x4*)((uint16_t*)sg.C + (size_t)(ti.row0 + r) * sg.N + ncol0 + ch * 8) = v;
  }
}

// One tile (or K-piece of a tile) in the full, half or quarter layout.
template <int BN, int WN, int EPI, int LAY, int WDT>
__device__ __forceinline__ void big_tile(const GemmArgs& a, const TileInfo& ti, const Seg& sg, const Work& wk,
                                         int ncol0, char* lds) {
  using C = BigCfg<BN, WN, LAY>;
  using M = BigMem<BN, WN, LAY, WDT>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: SGPR arithmetic
  const int K = sg.K;
  // this block's k-stages of the segment: all, piece k0num of s, or (router
  // logits) the blockIdx.y-th of ksplit ranges
  const int KT_all = K / BK;
  const int np = wk.s * a.ksplit, pi = wk.k0num * a.ksplit + (int)blockIdx.y;
  const int kt0 = pi * KT_all / np, kt1 = (pi + 1) * KT_all / np;

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
  const int a_plane = sg.a_prows * BK * 2;  // 0: row-major
  const int a_step = a_plane ? a_plane : BK * 2;  // bytes from one stage's slice to the next
  const __amdgpu_buffer_rsrc_t a_rsrc =
      a_plane ? uniform_rsrc(sg.A, (K / BK) * a_plane)
      : sg.amap ? uniform_rsrc(sg.A, a.a_map_rows * K * 2)
                : uniform_rsrc(sg.A + (size_t)ti.row0 * K * 2, ti.nrows * K * 2);
  uint32_t a_off[M::A_LOADS];
#pragma unroll
  for (int j = 0; j < M::A_LOADS; ++j) {
    const int s = (wave * M::A_LOADS + j) * 64 + lane;
    const int r = s / CH, c = (s % CH) ^ swz(r);
    const int rr = min(r, ti.nrows - 1);
    if (a_plane) {
      a_off[j] = (uint32_t)((ti.row0 + rr) * BK + c * 8) * 2u;
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

  // Stages past the end re-load the last stage into a buffer that is never
  // read again: every iteration then issues the same loads, the vmcnt waits
  // are constants and the refill can be scheduled between the MFMAs.
  // part 0 = the A loads of a stage, part 1 = its B loads
  auto issue_part = [&](int kt, int buf, int part) {
    char* st = lds + buf * M::STAGE_BYTES;
    const int ks = kt0 + min(kt, KT - 1);  // the stage's k-slice
    if (part == 0) {
#pragma unroll
      for (int j = 0; j < M::A_LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (lds_ptr_t)(st + (wave * M::A_LOADS + j) * 1024), 16, a_off[j], ks * a_step, 0, 0);
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

  f32x16 acc[C::TW][C::TA];
#pragma unroll
  for (int i = 0; i < C::TW; ++i)
#pragma unroll
    for (int j = 0; j < C::TA; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // Fragments of one k16 step: the wave's weight blocks and activation blocks.
  const int arow = wave_arow<BN, WN, LAY>(wave);
  struct Frags {
    bf16x8 w[C::TW], x[C::TA];
  };
  // A k16 step's k values for lane half h = lane / 32: bf16 weights use the
  // MFMA's own order (chunk 2 kk + h); fp8 weights use chunk 2 h + kk for both
  // operands -- the same permutation of k on both sides leaves the dot
  // products unchanged -- so one 16-byte read of a fp8 weight row holds the
  // lane's values for both k16 steps of the stage.
  u32x4 w8[C::TW];  // fp8: the stage's raw weight bytes (both steps)
  auto read_frags = [&](Frags& F, const char* L, int kk) {
    const int h = lane >> 5;
    const int c = (WDT == GD_FP8) ? 2 * h + kk : kk * 2 + h;
#pragma unroll
    for (int i = 0; i < C::TW; ++i) {
      const int wr = wave_wrow<BN, WN, LAY, EPI>(wave, i) + (lane & 31);
      if (WDT == GD_FP8) {
        if (kk == 0) w8[i] = *(const u32x4*)(L + M::A_BYTES + f8_off(wr, h));
        F.w[i] = kk == 0 ? e4m3x8_to_bf16(w8[i][0], w8[i][1]) : e4m3x8_to_bf16(w8[i][2], w8[i][3]);
      } else {
        F.w[i] = *(const bf16x8*)(L + M::A_BYTES + 2 * lds_off(wr, c));
      }
    }
#pragma unroll
    for (int j = 0; j < C::TA; ++j)
      F.x[j] = *(const bf16x8*)(L + 2 * lds_off(arow + j * 32 + (lane & 31), c));
  };
  auto mfmas = [&](const Frags& F) {
#pragma unroll
    for (int i = 0; i < C::TW; ++i)
#pragma unroll
      for (int j = 0; j < C::TA; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.w[i], F.x[j], acc[i][j], 0, 0, 0);
  };
  // Interleave the next step's fragment reads and half a stage refill with
  // this step's MFMAs, so issuing them never leaves the MFMA pipe idle.
  constexpr int NMF = C::TW * C::TA, NDS = C::TW + C::TA;
  auto interleave_refill = [&]() {
#pragma unroll
    for (int i = 0; i < NDS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NMF / (2 * NDS) > 0 ? NMF / (2 * NDS) : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (a half refill: <= NDS loads)
      __builtin_amdgcn_sched_group_barrier(0x008, NMF / (2 * NDS) > 0 ? NMF / (2 * NDS) : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // Pipeline over a ring of STAGES = 4 buffers, stage kt in buffer kt % 4.
  // Iteration kt computes stage kt in two k16 steps, each overlapping the
  // next step's fragment reads.  Between the steps it waits for its own loads
  // of stage kt+1 and passes the barrier, after which every wave holds its
  // stage-kt fragments in registers, so buffer kt % 4 is free.  Refills are
  // split to keep the address unit from bursting: the A half of stage kt+4 is
  // issued right after that barrier, its B half during step 0 of the next
  // iteration -- still two iterations before the stage is needed.  Stages
  // past the end re-load the last k-slice into buffers never read again, so
  // every wait is a constant.
  static_assert(STAGES == 4 && KK == 2, "pipeline is laid out for 4 stages of two k16 steps");
  issue_part(0, 0, 0); issue_part(0, 0, 1);
  issue_part(1, 1, 0); issue_part(1, 1, 1);
  issue_part(2, 2, 0); issue_part(2, 2, 1);
  issue_part(3, 3, 0);
  wait_vmcnt<2 * M::LOADS + M::A_LOADS>();  // stage 0 done
  barrier_only();

  Frags F[2];
  read_frags(F[0], lds, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const char* L = lds + (kt % STAGES) * M::STAGE_BYTES;
    // step 0: next fragments of this stage, B half of stage kt+3
    read_frags(F[1], L, 1);
    issue_part(kt + 3, (kt + 3) % STAGES, 1);
    mfmas(F[0]);
    interleave_refill();
    // step 1: stage kt+1 resident and stage kt retired everywhere, then the
    // A half of stage kt+4 into buffer kt % 4 and stage kt+1's first fragments
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    wait_vmcnt<2 * M::LOADS>();
    barrier_only();
    issue_part(kt + 4, kt % STAGES, 0);
    read_frags(F[0], lds + ((kt + 1) % STAGES) * M::STAGE_BYTES, 0);
    mfmas(F[1]);
    interleave_refill();
  }
  wait_vmcnt<0>();  // the re-loads past the end land before the block can exit

  if constexpr (EPI == EPI_BIAS_F32)  // router logits: never split (K ranges go to blockIdx.y)
    store_tile<C::TW, C::TA, WDT, EPI>(a, ti, sg, acc, arow, ncol0 + wave_col<BN, WN, LAY, EPI>(wave), lane);
  else
    finish_tile<BN, WN, EPI, LAY, WDT>(a, ti, sg, acc, ncol0, lds, wk.slot);
}
#endif

template <int BN, int WN, int EPI, int WDT>
__global__ __launch_bounds__(128 * WN, 1) void gemm_big_kernel(GemmArgs a, int n_tiles, int kt_plan,
                                                                int n_cu) {
  // device pass only: the host pass needs just the launch stub
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RING = STAGES * BigMem<BN, WN, 0, WDT>::STAGE_BYTES;
  constexpr int OUT = (EPI == EPI_BIAS_F32) ? 0 : OutTile<BN, EPI>::BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[RING > OUT ? RING : OUT];
  Work wk;
  if (!big_work(a, n_tiles, kt_plan, n_cu, BM, wk)) return;
  TileInfo ti;
  Seg sg;
  if (!tile_info(a, wk.mt, BM, ti, sg)) return;
  const int ncol0 = wk.nt * (EPI == EPI_SWIGLU ? BN / 2 : BN);
  if (ncol0 >= sg.N) return;
  switch (tile_layout(ti.nrows)) {
    case 2: big_tile<BN, WN, EPI, 2, WDT>(a, ti, sg, wk, ncol0, lds); break;
    case 1: big_tile<BN, WN, EPI, 1, WDT>(a, ti, sg, wk, ncol0, lds); break;
    default: big_tile<BN, WN, EPI, 0, WDT>(a, ti, sg, wk, ncol0, lds);
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
// A stage's 4 x 4 grid of 32x32 blocks runs in four quarters (weight half,
// activation half): (lo, lo), (lo, hi), (hi, hi), (hi, lo).  The fragments
// of the first quarter are in registers when the stage starts; the other
// halves of this stage are read during the first two quarters, then every
// wave passes the barrier (all of this stage read, the next stage landed)
// and the next stage's lo halves are read during the last two, so LDS reads
// stay spread over the MFMAs.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int BK8 = 64;            // k per stage of the fp8 x fp8 path
[[maybe_unused]] constexpr int SC_STAGES = 8;       // stages per 16-byte chunk of scales
[[maybe_unused]] constexpr int SC_BYTES = BM * 16;  // one chunk for every row of a tile

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

// Spread ND LDS reads and NV direct loads over the NM MFMAs of a quarter.
template <int NM, int ND, int NV>
__device__ __forceinline__ void sched_quarter() {
  constexpr int dpm = (ND + NM - 1) / NM, vpm = (NV + NM - 1) / NM;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (dpm > 0) __builtin_amdgcn_sched_group_barrier(0x100, dpm, 0);
    if (vpm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vpm, 0);
  }
}

#if defined(__HIP_DEVICE_COMPILE__)
template <int BN, int WN, int EPI, int LAY>
__device__ __forceinline__ void big_tile_fp8(const GemmArgs& a, const TileInfo& ti, const Seg& sg, const Work& wk,
                                             int ncol0, char* lds) {
  using C = BigCfg<BN, WN, LAY>;
  using M = BigMem<BN, WN, LAY, GD_BF16>;  // 64-byte rows on both operands: the bf16 stage geometry
  static_assert(C::NTHR == BM, "one scale row per thread");
  constexpr int TW2 = C::TW / 2, TA2 = C::TA / 2;
  static_assert(TW2 >= 1 && TA2 >= 1, "quarters");
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
    return frag(L + M::A_BYTES, wave_wrow<BN, WN, LAY, EPI>(wave, i) + (lane & 31));
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

  i32x8 WL[2][TW2], XL[2][TA2], WH[TW2], XH[TA2];
  // prologue: scale chunk 0, stages 0..2 and the A part of stage 3
  issue_scales(0);
  issue_part(0, 0, 0); issue_part(0, 0, 1);
  issue_part(1, 1, 0); issue_part(1, 1, 1);
  issue_part(2, 2, 0); issue_part(2, 2, 1);
  issue_part(3, 3, 0);
  wait_vmcnt<2 * M::LOADS + M::A_LOADS>();  // scale chunk 0 and stage 0 done
  barrier_only();
  read_scales(0);
#pragma unroll
  for (int i = 0; i < TW2; ++i) WL[0][i] = wfrag(lds, i);
#pragma unroll
  for (int j = 0; j < TA2; ++j) XL[0][j] = xfrag(lds, j);

  // Stage kt is in ring buffer kt % 4 = st % 4 (chunks are 8 stages), so
  // every LDS address below is a constant offset.  Waits and refills are
  // those of the bf16 pipeline; a scale chunk load adds one more load to
  // some waits' windows, which only makes them wait a little longer.
  for (int c = 0; c < NC; ++c) {
    static_for<0, SC_STAGES>([&](auto ST) {
      constexpr int st = decltype(ST)::value, p = st & 1;
      const int kt = c * SC_STAGES + st;
      if (kt >= KT) return;
      const char* L = lds + (st % STAGES) * M::STAGE_BYTES;
      const char* Ln = lds + ((st + 1) % STAGES) * M::STAGE_BYTES;
      int sb[C::TA];
#pragma unroll
      for (int j = 0; j < C::TA; ++j) sb[j] = (int)((SC[j][st >> 1] >> (16 * (st & 1) + 8 * h)) & 0xffu);
      if (st == 0) issue_scales(c + 1);
      // (lo, lo): read this stage's activation hi half; B part of stage kt+3
      issue_part(kt + 3, (st + 3) % STAGES, 1);
#pragma unroll
      for (int j = 0; j < TA2; ++j) XH[j] = xfrag(L, TA2 + j);
#pragma unroll
      for (int i = 0; i < TW2; ++i)
#pragma unroll
        for (int j = 0; j < TA2; ++j) mf(i, j, WL[p][i], XL[p][j], sb[j]);
      sched_quarter<TW2 * TA2, 2 * TA2, M::B_LOADS>();
      __builtin_amdgcn_sched_barrier(0);
      // (lo, hi): read this stage's weight hi half
#pragma unroll
      for (int i = 0; i < TW2; ++i) WH[i] = wfrag(L, TW2 + i);
#pragma unroll
      for (int i = 0; i < TW2; ++i)
#pragma unroll
        for (int j = 0; j < TA2; ++j) mf(i, TA2 + j, WL[p][i], XH[j], sb[TA2 + j]);
      sched_quarter<TW2 * TA2, 2 * TW2, 0>();
      __builtin_amdgcn_sched_barrier(0);
      // this stage read everywhere, stage kt+1 resident: A part of stage
      // kt+4 into this buffer
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      wait_vmcnt<2 * M::LOADS>();
      barrier_only();
      __builtin_amdgcn_sched_barrier(0);
      issue_part(kt + 4, st % STAGES, 0);
      // (hi, hi): next stage's weight lo half
#pragma unroll
      for (int i = 0; i < TW2; ++i) WL[p ^ 1][i] = wfrag(Ln, i);
#pragma unroll
      for (int i = 0; i < TW2; ++i)
#pragma unroll
        for (int j = 0; j < TA2; ++j) mf(TW2 + i, TA2 + j, WH[i], XH[j], sb[TA2 + j]);
      sched_quarter<TW2 * TA2, 2 * TW2, M::A_LOADS>();
      __builtin_amdgcn_sched_barrier(0);
      // (hi, lo): next stage's activation lo half (and, at a chunk's end,
      // the next chunk's scales)
#pragma unroll
      for (int j = 0; j < TA2; ++j) XL[p ^ 1][j] = xfrag(Ln, j);
      if (st == SC_STAGES - 1) read_scales(c + 1);
#pragma unroll
      for (int i = 0; i < TW2; ++i)
#pragma unroll
        for (int j = 0; j < TA2; ++j) mf(TW2 + i, j, WH[i], XL[p][j], sb[j]);
      sched_quarter<TW2 * TA2, 2 * TA2 + (st == SC_STAGES - 1 ? C::TA : 0), 0>();
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  wait_vmcnt<0>();  // the re-loads past the end land before the block can exit
  finish_tile<BN, WN, EPI, LAY, GD_FP8>(a, ti, sg, acc, ncol0, lds, wk.slot);
}
#endif

template <int BN, int WN, int EPI>
__global__ __launch_bounds__(128 * WN, 1) void gemm_big_fp8_kernel(GemmArgs a, int n_tiles, int kt_plan,
                                                                    int n_cu) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(OutTile<BN, EPI>::BYTES <= STAGES * BigMem<BN, WN, 0, GD_BF16>::STAGE_BYTES, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[STAGES * BigMem<BN, WN, 0, GD_BF16>::STAGE_BYTES +
                                                     2 * SC_BYTES];
  Work wk;
  if (!big_work(a, n_tiles, kt_plan, n_cu, BM, wk)) return;
  TileInfo ti;
  Seg sg;
  if (!tile_info(a, wk.mt, BM, ti, sg)) return;
  const int ncol0 = wk.nt * (EPI == EPI_SWIGLU ? BN / 2 : BN);
  if (ncol0 >= sg.N) return;
  switch (tile_layout(ti.nrows)) {
    case 2: big_tile_fp8<BN, WN, EPI, 2>(a, ti, sg, wk, ncol0, lds); break;
    case 1: big_tile_fp8<BN, WN, EPI, 1>(a, ti, sg, wk, ncol0, lds); break;
    default: big_tile_fp8<BN, WN, EPI, 0>(a, ti, sg, wk, ncol0, lds);
  }
#endif
}

// Fixup of the split tiles, one float4 of the pieces' register layout per
// work unit: unit ((i * TA + j) * 4 + g) * NTHR + t holds accumulator floats
// 4g..4g+3 of block (i, j) of GEMM thread t, i.e. four consecutive output
// columns of one row.  The unit's pieces are added in piece order (the same
// sum whichever block ran which piece), then the tile's epilogue is applied
// to those four columns.  SwiGLU units pair block i (u) with block i + TW/2
// (v).  Spreading units over many blocks keeps the reads in flight.
constexpr int kFixupChunks = 16;  // blocks per split tile
template <int BN, int WN, int EPI, int LAY, int WDT>
__device__ __forceinline__ void fixup_units(const GemmArgs& a, const TileInfo& ti, const Seg& sg, int ncol0,
                                            int first_slot, int s) {
  using C = BigCfg<BN, WN, LAY>;
  constexpr int NT = 128 * WN;  // threads of the GEMM block
  constexpr int TWO = (EPI == EPI_SWIGLU) ? C::TW / 2 : C::TW;
  constexpr int UNITS = NT * TWO * C::TA * 4;
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
    const int g = r & 3, j = (r >> 2) % C::TA, i = (r >> 2) / C::TA;
    const int wave = t >> 6, lane = t & 63;
    const int row = wave_arow<BN, WN, LAY>(wave) + j * 32 + (lane & 31);
    if (row >= ti.nrows) continue;
    const int n = ncol0 + wave_col<BN, WN, LAY, EPI>(wave) + i * 32 + g * 8 + (lane >> 5) * 4;
    float o[4];
    const float4 x = sum(((i * C::TA + j) * 4 + g) * NT + t);
    if (EPI == EPI_SWIGLU) {
      const float4 y = sum((((i + C::TW / 2) * C::TA + j) * 4 + g) * NT + t);
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

// Blocks (split tile, chunk).
template <int BN, int WN, int EPI, int WDT>
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
      case 2: fixup_units<BN, WN, EPI, 2, WDT>(a, ti, sg, ncol0, blockIdx.x * p.s, p.s); break;
      case 1: fixup_units<BN, WN, EPI, 1, WDT>(a, ti, sg, ncol0, blockIdx.x * p.s, p.s); break;
      default: fixup_units<BN, WN, EPI, 0, WDT>(a, ti, sg, ncol0, blockIdx.x * p.s, p.s);
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
  const int n_slots = a.tile_table ? a.n_slots : (a.rows + BM - 1) / BM;
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
  if constexpr (FP8ACT)
    hipLaunchKernelGGL((gemm_big_fp8_kernel<BN, WN, EPI>), dim3(nb), dim3(128 * WN), 0, s, a, n_tiles, kt_plan,
                       n_cu);
  else
    hipLaunchKernelGGL((gemm_big_kernel<BN, WN, EPI, WDT>), dim3(nb, a.ksplit), dim3(128 * WN), 0, s, a,
                       n_tiles, kt_plan, n_cu);
  if (n_cu > 0)
    hipLaunchKernelGGL((gemm_big_fixup_kernel<BN, WN, EPI, WDT>), dim3(n_cu / 2, kFixupChunks), dim3(256),
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
