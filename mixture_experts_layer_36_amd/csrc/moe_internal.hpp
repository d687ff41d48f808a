// Internal interfaces between the C ABI (moe_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- device utils
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> packed bf16 pair (lo in bits 0..15): gfx950's pair
// conversion (v_cvt_pk_bf16_f32), one instruction.  It rounds to nearest,
// ties to even, like f32_to_bf16: a probe over 8.4 M bit patterns (ties,
// f32 subnormals, the largest finite values, infinities) matched it bit for
// bit; only a NaN's payload bits may differ (a NaN stays a NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// OCP E4M3 byte -> bf16 bits (exact: every E4M3 value is a bf16 value).
// Normal: exponent rebias 7 -> 127, mantissa moves up 4 bits.
// Subnormal (exp 0): value m * 2^-9, built from the integer m.
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 8;
  const uint32_t em = b & 0x7fu;
  uint32_t mag;
  if (em >= 0x08u) {
    mag = (em << 4) + (120u << 7);
  } else {
    mag = __float_as_uint((float)em * 0.001953125f) >> 16;  // m * 2^-9, exact
  }
  return sign | mag;
}

// Four OCP E4M3 codes (bytes 0..3 of w) -> their bf16 bits, two per word
// (bytes 0, 1 in word 0), exactly: gfx950's packed scaled conversion with a
// scale of 1.0.  Whole pairs are bit-cast: clang miscompiles a bit cast of
// one component of such a vector (it takes the first component).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16_bits(uint32_t w) {
  u32x2 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return o;
}

// ------------------------------------------------------------------ launchers
struct RouteSelectArgs {
  const float* z;        // [ksplit][T][E] partial router logits (bias in part 0)
  int ksplit;
  int T, E, k, score, renorm, n_group, topk_group;
  int32_t* topk_idx;     // [T][k]
  float* topk_w;         // [T][k]
  // Optional (nullable): the token's eligible experts of rank k .. 2k-1 (-1
  // past the eligible ones) and their gates (score / sum of the top-k scores
  // when renorm, else the score): the reroute candidates.
  int32_t* cand_idx;     // [T][k]
  float* cand_w;         // [T][k]
};
hipError_t launch_route_select(const RouteSelectArgs& a, hipStream_t s);

// The whole router in one kernel for few experts: logits x Wr^T + b, scores,
// top-k, gates (and reroute candidates), with the selection rules of
// route_select.  Taken when router_fused_ok().
struct RouterFusedArgs {
  const void* x;         // [T][d] bf16
  const void* w_router;  // [E][d] bf16
  const float* bias;     // [E] or NULL
  int T, d, E, k, score, renorm;
  int32_t* topk_idx;     // [T][k]
  float* topk_w;         // [T][k]
  int32_t* cand_idx;     // [T][k] or NULL
  float* cand_w;
};
bool router_fused_ok(int T, int d, int E, int k, int n_group, int act);
hipError_t launch_router_fused(const RouterFusedArgs& a, hipStream_t s);

// Dispatch: assignments are processed in chunks of dispatch_chunk(n_assign)
// (a power of two in [kMinDispatchChunk, kMaxDispatchChunk], about 64 chunks:
// one wavefront walks a chunk, the scan walks the chunks); workspaces are
// sized for the smallest chunk.
constexpr int kMinDispatchChunk = 256, kMaxDispatchChunk = 1024;
inline int dispatch_chunk(long long n_assign) {
  int c = kMinDispatchChunk;
  while (c < kMaxDispatchChunk && (long long)c * 64 < n_assign) c *= 2;
  return c;
}
struct DispatchArgs {
  const int32_t* topk_idx;  // [T*k]
  int n_assign, E, k;
  int32_t* chunk_cnt;       // [n_chunks][E] workspace (counts, then bases)
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* perm_token;      // [n_assign]
  int32_t* inv_pos;         // [n_assign]
  int cap;                  // slots per expert (INT32_MAX: dropless)
  int chunk;                // assignments per chunk (set by the launchers)
};
hipError_t launch_dispatch_index(const DispatchArgs& a, hipStream_t s);

// Capacity with overflow rerouted: the two-pass dispatch.  Inputs: the
// DispatchArgs above (cap < INT32_MAX), the router's gates and the reroute
// candidates; workspace: chunk_cnt2 [n_chunks][E], rel and target [n_assign].
// Output besides counts/offsets/perm_token/inv_pos: gate [n_assign], the gate
// of the copy that serves each assignment (combine reads it as its topk_w).
struct RerouteArgs {
  const float* topk_w;      // [T*k]
  const int32_t* cand_idx;  // [T*k]
  const float* cand_w;      // [T*k]
  int32_t* chunk_cnt2;
  int32_t* rel;             // rank of each assignment within its own expert
  int32_t* target;          // candidate offered to an overflowed assignment, else -1
  float* gate;              // [T*k]
};
hipError_t launch_dispatch_reroute(const DispatchArgs& a, const RerouteArgs& r, hipStream_t s);

// rows[e] = offsets[e+1] - offsets[e], e < E.
hipError_t launch_segment_rows(const int32_t* offsets, int E, int32_t* rows, hipStream_t s);

// x_perm[p] = x[perm_token[p]] for p < min(rows, *rows_dev) (rows_dev: device
// row count, nullable), rows of row_bytes (multiple of 16).
hipError_t launch_gather_rows(const void* x, const int32_t* perm_token, int rows, const int32_t* rows_dev,
                              int row_bytes, void* x_perm, hipStream_t s);
// The same rows into the K-blocked planes of GemmArgs::a_blk (P = rows) of
// width pw = 32 or 64: bf16, d a multiple of pw; perm_token NULL copies x's
// rows in order.
hipError_t launch_gather_rows_blocked(const void* x, const int32_t* perm_token, int rows, const int32_t* rows_dev,
                                      int d, int pw, void* x_perm, hipStream_t s);

// The block-scaled E4M3 dispatch payload (fp8_payload.hip): bf16 rows cut
// into blocks of 32 elements, each block one E8M0 scale 2^s (s smallest with
// amax <= 448 * 2^s, 0 for an all-zero block) and E4M3 codes of x / 2^s
// rounded to nearest even.  Row p of the output reads source row perm[p]
// (perm NULL: row p) for p < min(rows, *rows_dev) (rows_dev nullable).
// deq == NULL: codes [rows][d] and scales [rows][sstride] are written;
// otherwise the dequantised values as bf16 rows [rows][d] go to deq.
constexpr int kFp8Block = 32;
struct Fp8PayloadArgs {
  const void* x;            // bf16 source rows [.][d]
  const int32_t* perm;
  int rows;
  const int32_t* rows_dev;
  int d;
  uint8_t* codes;
  uint8_t* scales;
  int sstride;              // bytes between scale rows (>= d / 32)
  void* deq;
};
hipError_t launch_fp8_payload(const Fp8PayloadArgs& a, hipStream_t s);
// Payload codes [rows][d] + scales [rows][sstride] -> bf16 rows [rows][d]
// (exact), rows p < min(rows, *rows_dev).
hipError_t launch_fp8_dequant(const uint8_t* codes, const uint8_t* scales, int sstride, int rows,
                              const int32_t* rows_dev, int d, void* out, hipStream_t s);

// Combine.
struct CombineArgs {
  const void* y_perm;
  const int32_t* inv_pos;
  const float* topk_w;
  const void* shared_y;  // nullable
  void* out;
  int T, d, k, act;      // act: 0 f32, 1 bf16
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// Grouped GEMM over ragged expert segments.
//   C[m][n] = epilogue( sum_k A[m][k] * B_e[n][k] )
// A rows are activations (row-major, K contiguous); B_e is the weight matrix
// of the segment's expert (out x in, K contiguous).
enum GemmEpilogue { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_BIAS_F32 = 2 };
enum GemmDtype { GD_F32 = 0, GD_BF16 = 1, GD_FP8 = 2 };  // act GD_FP8: the block-scaled payload

struct GemmArgs {
  const void* A;               // [rows][K] activations (a_map: [a_map_rows][K])
  int rows;                    // rows of the routed segments
  // Optional row map of the routed segments: buffer row p reads A row
  // a_map[p] (the fused dispatch gather: A = x, a_map = perm_token).
  const int32_t* a_map;
  int a_map_rows;              // rows of A when a_map is set
  int E;                       // routed segments (experts); 0 or 1: one segment
  const int32_t* tile_table;   // [n_slots + 1]: (segment << 21 | m-tile in segment) or -1, then
                               // the number of real m-tiles; NULL: one segment of `rows`
  const int32_t* offsets;      // [E+1] segment starts (with tile_table)
  int n_slots;                 // m-tile slots in the grid
  const void* B0;              // [E][N][K] weights (gate projection W1 for SwiGLU)
  const void* B1;              // [E][N][K] up projection W3 (SwiGLU only)
  const float* s0;             // [E][N] fp8 scales of B0 (NULL otherwise)
  const float* s1;             // [E][N] fp8 scales of B1
  const float* bias;           // [N] (EPI_BIAS_F32)
  int N;                       // output columns (h columns for SwiGLU)
  int K;
  void* C;                     // [rows][N] output; EPI_BIAS_F32: [ksplit][rows][N] partial sums
  int act;                     // GemmDtype of A (F32, BF16, or FP8: E4M3 codes with a_scales) and
                               // of C (F32 for F32, else BF16); EPI_BIAS_F32 stores f32
  int wdt;                     // GemmDtype of B
  int epi;                     // GemmEpilogue
  int ksplit;                  // EPI_BIAS_F32: K is split into ksplit equal ranges (>= 1)
  // Optional extra segment E (the shared expert): sh_rows rows of shA in
  // order, its own weights (wdt == act), output and sizes.
  int sh_rows;                 // 0: none
  const void* shA;
  const void* shB0;
  const void* shB1;
  void* shC;
  int shN, shK;
  // Prefill kernel only: fp32 slots for the K-split pieces of the tiles left
  // over after the last full wave of tiles (NULL / 0: never split).
  float* partial;
  int partial_slots;
  // act == GD_FP8: E8M0 scales of A, one byte per 32 k values, rows of
  // a_sstride bytes (a multiple of 16), indexed like A's rows.
  const uint8_t* a_scales;
  int a_sstride;
  // Prefill kernel only, bf16: K-blocked operands.  A K-blocked matrix of P
  // rows and K columns is K/W planes of [P][W] elements (plane width W = 32,
  // or 64 for the wide form), element (r, k) at (k / W) * P * W + r * W +
  // k % W, so the W-column slice of a tile's rows is one contiguous run.
  // a_blk: 0, or A in this layout with W = 32 (1) or 64 (2, SwiGLU only, K a
  // multiple of 64), P = rows, or, with a row map, P = a_map_rows (the map
  // indexes the planes' rows); sh_a_blk: likewise the extra segment's shA
  // with P = sh_rows.  c_blk (SwiGLU only): C with W = 32 and P = rows, and
  // shC with P = sh_rows.  Each matrix must stay under 2^31 bytes.
  int a_blk;
  int sh_a_blk;
  int c_blk;
  // Routed weights B0/B1 in the K-blocked layout (P = N per expert matrix);
  // the extra segment's weights are row-major.  bf16 / fp8 weights only.
  int b_blk;
  // Prefill kernel with a tile table: room for sched_cap block records of
  // kSchedInts ints.  A schedule kernel resolves each block's tile (m-tile,
  // n-tile, K-piece, segment, rows) before the GEMM launch, and each GEMM
  // block then reads its record instead of deriving it.  NULL, or fewer
  // records than blocks: every block derives its own.
  int32_t* sched;
  int sched_cap;
  // Prefill kernel without a tile table (the router logits): rows per m-tile,
  // 256 or 128 (0: 256).
  int m_tile;
};
constexpr int kSchedInts = 8;

// Row-major [mats][rows][cols] -> K-blocked [mats][cols/32][rows][32] of
// elem_bytes-byte elements (1 or 2).
hipError_t launch_pack_kblocked(const void* src, int64_t mats, int rows, int cols, int elem_bytes, void* dst,
                                hipStream_t s);

// Bytes of one partial-sum slot (one 256 x 256 tile of fp32 accumulators) and
// the slots a launch may use (at most one per compute unit).
constexpr size_t kPartialSlotBytes = 256 * 256 * 4;
constexpr int kPartialSlots = 256;

// Rows per m-tile the grouped GEMM uses for this problem (the tile table must
// be built with the same value).
int gemm_block_m(const GemmArgs& a);
// Upper bound of m-tile slots for `rows` rows in E segments plus an extra
// segment of sh_rows rows.
int gemm_max_slots(int rows, int E, int block_m, int sh_rows);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// Whether launch_gemm takes act == GD_FP8 for this problem (E4M3 weights,
// the SwiGLU epilogue, no extra segment, a prefill-sized grouped GEMM).
bool gemm_fp8_act_ok(const GemmArgs& a);

// Tile tables for up to two tile heights from segment offsets.
struct TileTableArgs {
  const int32_t* offsets;  // [E+1]
  int E;
  int sh_rows;             // rows of the extra segment E (0: none)
  int bm0, n_slots0;
  int32_t* table0;         // [n_slots0 + 1]
  int bm1, n_slots1;       // bm1 = 0: only one table
  int32_t* table1;
};
hipError_t launch_tile_tables(const TileTableArgs& a, hipStream_t s);

}  // namespace moe
