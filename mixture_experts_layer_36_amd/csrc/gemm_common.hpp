// Shared pieces of the grouped-GEMM kernels: tile table decoding, XCD-aware
// block mapping and the MFMA-layout epilogues.
#pragma once

#include "moe_internal.hpp"

namespace moe {

constexpr int kTableExpertShift = 21;
constexpr int kTableTileMask = (1 << kTableExpertShift) - 1;

struct TileInfo {
  int e, row0, nrows;
};

// Operands of the segment a tile belongs to.
struct Seg {
  const char* A;            // activation rows of the segment's buffer (row 0 = buffer row 0)
  const char* B0;           // this expert's weight matrices
  const char* B1;
  const float* s0;          // this expert's per-channel scales (fp8) or NULL
  const float* s1;
  char* C;
  int N, K;
  const int32_t* amap;      // routed rows through the row map (NULL: rows in order)
  int a_prows;              // A K-blocked with planes of a_prows rows (0: row-major)
  int a_wide;               // ... of 64 columns (else 32)
  int c_prows;              // C K-blocked likewise (0: row-major)
  int b_blk;                // B0/B1 K-blocked with planes of N rows
};

// A row of segment row `r` (tile-relative row r of a tile starting at row0).
__device__ __forceinline__ int a_row(const Seg& sg, int row0, int r) {
  return sg.amap ? sg.amap[row0 + r] : row0 + r;
}

__device__ __forceinline__ int dtype_bytes(int dt) { return dt == GD_F32 ? 4 : dt == GD_BF16 ? 2 : 1; }

// The operands of segment ti.e (a.E with a tile table: the extra, shared
// segment), from the arguments alone.
__device__ __forceinline__ void tile_seg(const GemmArgs& a, const TileInfo& ti, Seg& sg) {
  if (a.tile_table != nullptr && ti.e == a.E) {  // the extra (shared) segment
    sg.A = (const char*)a.shA;
    sg.B0 = (const char*)a.shB0;
    sg.B1 = (const char*)a.shB1;
    sg.s0 = sg.s1 = nullptr;
    sg.C = (char*)a.shC;
    sg.N = a.shN;
    sg.K = a.shK;
    sg.amap = nullptr;
    sg.a_prows = a.sh_a_blk ? a.sh_rows : 0;
    sg.a_wide = a.sh_a_blk == 2;
    sg.c_prows = a.c_blk ? a.sh_rows : 0;
    sg.b_blk = 0;
    return;
  }
  const size_t woff = (size_t)ti.e * a.N * a.K * dtype_bytes(a.wdt);
  sg.A = (const char*)a.A;
  sg.B0 = (const char*)a.B0 + woff;
  sg.B1 = a.B1 ? (const char*)a.B1 + woff : nullptr;
  sg.s0 = a.s0 ? a.s0 + (size_t)ti.e * a.N : nullptr;
  sg.s1 = a.s1 ? a.s1 + (size_t)ti.e * a.N : nullptr;
  sg.C = (char*)a.C;
  sg.N = a.N;
  sg.K = a.K;
  sg.amap = a.a_map;
  sg.a_prows = a.a_blk ? (a.a_map ? a.a_map_rows : a.rows) : 0;
  sg.a_wide = a.a_blk == 2;
  sg.c_prows = a.c_blk ? a.rows : 0;
  sg.b_blk = a.b_blk;
}

// m-tile slot -> (segment, first row, rows in the tile); false for empty
// slots.
__device__ __forceinline__ bool tile_rows(const GemmArgs& a, int mt, int BM, TileInfo& ti) {
  int tile;
  if (a.tile_table == nullptr) {
    ti.e = 0;
    tile = mt;
  } else {
    const int code = a.tile_table[mt];
    if (code < 0) return false;
    ti.e = code >> kTableExpertShift;
    tile = code & kTableTileMask;
  }
  if (a.tile_table != nullptr && ti.e == a.E) {  // the extra (shared) segment
    ti.row0 = tile * BM;
    ti.nrows = min(BM, a.sh_rows - ti.row0);
  } else if (a.tile_table == nullptr) {
    ti.row0 = tile * BM;
    ti.nrows = min(BM, a.rows - ti.row0);
  } else {
    const int lo = a.offsets[ti.e], hi = a.offsets[ti.e + 1];
    ti.row0 = lo + tile * BM;
    ti.nrows = min(BM, hi - ti.row0);
  }
  return ti.nrows > 0;
}

// m-tile slot -> its rows and operands; false for empty slots.
__device__ __forceinline__ bool tile_info(const GemmArgs& a, int mt, int BM, TileInfo& ti, Seg& sg) {
  if (!tile_rows(a, mt, BM, ti)) return false;
  tile_seg(a, ti, sg);
  return true;
}

// Number of real m-tiles: the tile table stores it after its n_slots entries.
__device__ __forceinline__ int real_mtiles(const GemmArgs& a, int BM) {
  return a.tile_table ? a.tile_table[a.n_slots] : (a.rows + BM - 1) / BM;
}

// Block -> (m-tile slot, n-tile).  Blocks are dealt round-robin to the 8 XCDs
// (block b runs on XCD b % 8), so XCD x owns an equal contiguous share of the
// real tiles; within it tiles go in groups of kGroupM m-slots x all n-tiles
// (m fastest), so the blocks an XCD runs at once share A and B tiles in its
// L2.  gridDim.x is a multiple of 8 and covers the upper bound of tiles;
// blocks beyond the real count exit.
constexpr int kGroupM = 4;
// Tile L of the grouped order -> (m-tile slot, n-tile).
__device__ __forceinline__ void tile_coords(int L, int m_real, int n_tiles, int& mt, int& nt) {
  const int g = L / (kGroupM * n_tiles), within = L % (kGroupM * n_tiles);
  const int gm = min(kGroupM, m_real - g * kGroupM);
  mt = g * kGroupM + within % gm;
  nt = within / gm;
}
// Block (XCD x, index i on it) of an equal per-XCD share of the first Rw
// tiles of the grouped order -> its tile L.  Whole groups go to the XCDs in
// turn (super-groups of 8 groups: XCD x takes the x-th), so the 8 blocks of
// one dispatch round sit at the same place in 8 neighbouring groups --
// usually tiles of the same expert and kind, of equal duration -- while the
// blocks an XCD runs at once still share operands in its L2; tiles past the
// last whole super-group are dealt in turn one by one.  False past Rw.
__device__ __forceinline__ bool xcd_tile(int x, int i, int Rw, int n_tiles, int& L) {
  const int G = kGroupM * n_tiles, SG = 8 * G;
  const int ns = Rw / SG;
  if (i < ns * G) {
    L = (i / G) * SG + x * G + i % G;
    return true;
  }
  L = ns * SG + (i - ns * G) * 8 + x;
  return L < Rw;
}
__device__ __forceinline__ void block_coords(int m_real, int n_tiles, int& mt, int& nt) {
  const int per_xcd = (gridDim.x >> 3);
  const int R = m_real * n_tiles;
  const int share = (R + 7) >> 3;
  const int i = blockIdx.x >> 3;
  const int L = (blockIdx.x & 7) * share + i;
  mt = -1;
  if (i >= share || L >= R || i >= per_xcd) return;
  tile_coords(L, m_real, n_tiles, mt, nt);
}

// silu(u) = u * sigmoid(u) with the hardware exp2 and reciprocal: relative
// error ~1e-6, far below the bf16 rounding applied to the result.
__device__ __forceinline__ float silu(float u) {
  return u * __builtin_amdgcn_rcpf(1.f + __expf(-u));
}

// Epilogue of a wave's TW x TA grid of BHxBH MFMA blocks (BH = 32 or 16)
// computed as (weight rows) x (activation rows).  In block (i, j), lane l
// holds weight rows g*8 + (l/BH)*4 + q (q = 0..3, run g < BH*BH/256) of
// activation row l % BH, i.e. runs of 4 consecutive output columns.
//   col0: first output column of this wave's weight rows
//   SwiGLU: blocks i < TW/2 are W1 (u), blocks i + TW/2 the matching W3 (v).
template <int TW, int TA, int WDT, int EPI, int BH = 32, class AV = f32x16>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const TileInfo& ti, const Seg& sg,
                                           AV (&acc)[TW][TA], int row_base, int col0,
                                           int lane) {
  constexpr int G = BH * BH / 256;  // runs per lane and block
  const int r_in = lane % BH;
  const bool scaled = WDT == GD_FP8 && sg.s0 != nullptr;
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < TW / 2; ++i) {
      // fp8 per-output-channel scales of this block's columns: one 16-byte
      // load per run of 4 columns, shared by all activation blocks
      float4 su[G], sv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int n = col0 + i * BH + g * 8 + (lane / BH) * 4;
        if (scaled) {
          su[g] = *(const float4*)(sg.s0 + n);
          sv[g] = *(const float4*)(sg.s1 + n);
        }
      }
#pragma unroll
      for (int j = 0; j < TA; ++j) {
        const int lrow = row_base + j * BH + r_in;
        if (lrow >= ti.nrows) continue;
        const size_t row = (size_t)(ti.row0 + lrow);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int n = col0 + i * BH + g * 8 + (lane / BH) * 4;
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float u = acc[i][j][g * 4 + q];
            float v = acc[i + TW / 2][j][g * 4 + q];
            if (scaled) {
              u *= su[g][q];
              v *= sv[g][q];
            }
            hv[q] = silu(u) * v;
          }
          u32x2 o;
          o[0] = pack_bf16x2(hv[0], hv[1]);
          o[1] = pack_bf16x2(hv[2], hv[3]);
          *(u32x2*)((uint16_t*)sg.C + row * sg.N + n) = o;
        }
      }
    }
  } else if (EPI == EPI_STORE) {
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      float4 sc[G];
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (scaled) sc[g] = *(const float4*)(sg.s0 + col0 + i * BH + g * 8 + (lane / BH) * 4);
#pragma unroll
      for (int j = 0; j < TA; ++j) {
        const int lrow = row_base + j * BH + r_in;
        if (lrow >= ti.nrows) continue;
        const size_t row = (size_t)(ti.row0 + lrow);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int n = col0 + i * BH + g * 8 + (lane / BH) * 4;
          float yv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            yv[q] = acc[i][j][g * 4 + q];
            if (scaled) yv[q] *= sc[g][q];
          }
          u32x2 o;
          o[0] = pack_bf16x2(yv[0], yv[1]);
          o[1] = pack_bf16x2(yv[2], yv[3]);
          *(u32x2*)((uint16_t*)sg.C + row * sg.N + n) = o;
        }
      }
    }
  } else {  // EPI_BIAS_F32: router logits (partial sums of one K range)
#pragma unroll
    for (int j = 0; j < TA; ++j) {
      const int lrow = row_base + j * BH + r_in;
      if (lrow >= ti.nrows) continue;
      const size_t row = (size_t)(ti.row0 + lrow);
#pragma unroll
      for (int i = 0; i < TW; ++i) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int n = col0 + i * BH + g * 8 + (lane / BH) * 4;
          float* zr = (float*)sg.C + ((size_t)blockIdx.y * a.rows + row) * sg.N + n;
          if ((sg.N & 3) == 0 && n + 3 < sg.N) {  // whole run, 16-byte aligned
            float4 z = make_float4(acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                                   acc[i][j][g * 4 + 3]);
            if (a.bias && blockIdx.y == 0) {
              z.x += a.bias[n];
              z.y += a.bias[n + 1];
              z.z += a.bias[n + 2];
              z.w += a.bias[n + 3];
            }
            *(float4*)zr = z;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (n + q < sg.N) {
                float z = acc[i][j][g * 4 + q];
                if (a.bias && blockIdx.y == 0) z += a.bias[n + q];
                zr[q] = z;
              }
            }
          }
        }
      }
    }
  }
}

// Widest output among the segments of a launch.
inline int gemm_max_cols(const GemmArgs& a) { return (a.sh_rows > 0 && a.shN > a.N) ? a.shN : a.N; }

// Launchers of the individual kernel families (gemm.hip, gemm_big.hip,
// gemm_decode.hip).
hipError_t launch_gemm_big(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_decode(const GemmArgs& a, hipStream_t s);

}  // namespace moe
