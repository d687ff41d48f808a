// Grouped GEMM over ragged expert segments, with the SwiGLU, plain-store and
// router-bias epilogues.
//
// The experts of an MoE layer run as grouped GEMMs ("Tensor vs Expert vs Data
// Parallelism for MoE Serving", section "Deeper Analysis", Figure 2; "Expert
// Parallelism for MoE Serving", section "The Future of Expert Parallelism for
// MoE Serving").  Expert e owns rows [offsets[e], offsets[e+1]) of the
// expert-contiguous activation buffer; a device-built tile table maps each
// m-tile slot of the grid to (expert, m-tile), so the host never reads counts.
//
// bf16 / fp8-weight path (gfx950 MFMA):
//   * block tile BM activation rows x BN weight rows x BK=64, 4 wavefronts in
//     a 2x2 grid, LDS double-buffered, 16-byte chunks XOR-swizzled by row so
//     the MFMA operand reads spread over the LDS banks;
//   * v_mfma_f32_32x32x16_bf16 with the WEIGHT rows as the MFMA row operand
//     and activation rows as its column operand: each lane then owns runs of
//     4 consecutive output columns of one activation row, which become 8-byte
//     (bf16) or 16-byte (fp32) stores;
//   * fp8 (OCP E4M3) weights are widened to bf16 exactly while being staged
//     (gfx950's packed scaled conversion, two codes per instruction)
//     into LDS; the per-output-channel scale multiplies the fp32 accumulator
//     in the epilogue, so y = s_n * sum_k x_k q_nk exactly as dequantised;
//   * SwiGLU: each wavefront's weight rows are half W1 rows and half W3 rows
//     of the same output columns, so u and v meet in one lane and
//     h = silu(u) * v is formed before the store.
// fp32 path: an LDS-tiled FMA kernel (small layers; exact fp32 arithmetic).
//
// Grid: m-tile slots x n-tiles, remapped so that each XCD (blocks are dealt
// round-robin to the 8 XCDs) runs a contiguous run of slots of one n-tile and
// its L2 holds the weight tile those slots share.
#include "gemm_common.hpp"

namespace moe {
namespace {

// ============================================================== MFMA kernel
template <int BM, int BN, int WDT, int EPI>
struct MfmaCfg {
  static constexpr int BK = 64;
  static constexpr int WM = 2, WN = 2, NTHR = 256;
  static constexpr int RA = BM / WM;        // activation rows per wave
  static constexpr int RW = BN / WN;        // weight rows per wave
  static constexpr int TA = RA / 32, TW = RW / 32;
  static constexpr int A_CHUNKS = BM * BK / 8 / NTHR;  // 16-byte chunks per thread
  static constexpr int B_CHUNKS = (WDT == GD_FP8) ? BN * BK / 16 / NTHR : BN * BK / 8 / NTHR;
  static constexpr int NCOL = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns per tile
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");
  static_assert(EPI != EPI_SWIGLU || TW % 2 == 0, "SwiGLU needs paired weight blocks");
};

__device__ __forceinline__ int swz(int row, int chunk) {  // element offset in a 64-wide row
  return row * 64 + ((chunk ^ (row & 7)) << 3);
}

template <int BM, int BN, int WDT, int EPI>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs a, int n_slots, int n_tiles) {
  using C = MfmaCfg<BM, BN, WDT, EPI>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][(BM + BN) * C::BK];

  int mt, nt;
  block_coords(real_mtiles(a, BM), n_tiles, mt, nt);
  if (mt < 0) return;
  TileInfo ti;
  Seg sg;
  if (!tile_info(a, mt, BM, ti, sg)) return;
  const int ncol0 = nt * C::NCOL;
  if (ncol0 >= sg.N) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int K = sg.K;
  // split-K (router logits): this block sums k in [k_begin, k_begin + kspan)
  const int kspan = K / a.ksplit, k_begin = blockIdx.y * kspan;

  // ---- global source pointers of this thread's chunks (k offset added per tile)
  const uint16_t* a_src[C::A_CHUNKS];
  int a_dst[C::A_CHUNKS];
#pragma unroll
  for (int j = 0; j < C::A_CHUNKS; ++j) {
    const int q = tid + j * C::NTHR;
    const int r = q >> 3, c = q & 7;
    const int rr = min(r, ti.nrows - 1);
    a_src[j] = (const uint16_t*)sg.A + (size_t)a_row(sg, ti.row0, rr) * K + k_begin + c * 8;
    a_dst[j] = swz(r, c);
  }
  const uint8_t* b_src[C::B_CHUNKS];
  int b_dst[C::B_CHUNKS];
#pragma unroll
  for (int j = 0; j < C::B_CHUNKS; ++j) {
    const int q = tid + j * C::NTHR;
    int r, c;  // LDS row, first LDS chunk
    if (WDT == GD_FP8) { r = q >> 2; c = (q & 3) * 2; } else { r = q >> 3; c = q & 7; }
    const char* base;
    int n;
    if (EPI == EPI_SWIGLU) {
      const int half = C::RW / 2;
      const int w = r / C::RW, rr = r % C::RW;
      base = (rr < half) ? sg.B0 : sg.B1;
      n = ncol0 + w * half + (rr % half);
    } else {
      base = sg.B0;
      n = min(ncol0 + r, sg.N - 1);
    }
    const int esz = (WDT == GD_FP8) ? 1 : 2;
    // K-blocked weights: element (n, k) at (k / 32) * N * 32 + n * 32 + k % 32
    // (the chunk of 8 or 16 elements at k = c * 8 stays in one plane)
    b_src[j] = (const uint8_t*)base +
               (sg.b_blk ? (size_t)(c * 8 / 32) * sg.N * 32 + (size_t)n * 32 + (c * 8) % 32
                         : (size_t)n * K + k_begin + c * 8) * esz;
    b_dst[j] = BM * C::BK + swz(r, c);
  }
  // elements from one k tile's slice to the next: K-blocked, k0 columns
  // start k0 / 32 planes of N * 32 further
  const size_t b_kstride = sg.b_blk ? (size_t)sg.N : 1;

  u32x4 ra[C::A_CHUNKS], rb[C::B_CHUNKS];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < C::A_CHUNKS; ++j) ra[j] = *(const u32x4*)(a_src[j] + k0);
#pragma unroll
    for (int j = 0; j < C::B_CHUNKS; ++j)
      rb[j] = *(const u32x4*)(b_src[j] + (size_t)k0 * b_kstride * (WDT == GD_FP8 ? 1 : 2));
  };
  auto store = [&](int buf) {
    __bf16* L = lds[buf];
#pragma unroll
    for (int j = 0; j < C::A_CHUNKS; ++j) *(u32x4*)(L + a_dst[j]) = ra[j];
#pragma unroll
    for (int j = 0; j < C::B_CHUNKS; ++j) {
      if (WDT == GD_FP8) {
        // 16 e4m3 bytes -> two chunks of 8 bf16; the second chunk is c+1
        u32x4 lo, hi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u32x2 pp = e4m3x4_to_bf16_bits(rb[j][w]);
          const uint32_t p0 = pp[0], p1 = pp[1];
          if (w < 2) { lo[2 * w] = p0; lo[2 * w + 1] = p1; } else { hi[2 * w - 4] = p0; hi[2 * w - 3] = p1; }
        }
        const int off = b_dst[j] - BM * C::BK;
        const int r = off >> 6;
        const int c = ((off & 63) >> 3) ^ (r & 7);
        *(u32x4*)(L + BM * C::BK + swz(r, c)) = lo;
        *(u32x4*)(L + BM * C::BK + swz(r, c + 1)) = hi;
      } else {
        *(u32x4*)(L + b_dst[j]) = rb[j];
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

  const int KT = kspan / C::BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load((kt + 1) * C::BK);
    const __bf16* L = lds[cur];
#pragma unroll
    for (int kk = 0; kk < C::BK / 16; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      bf16x8 fw[C::TW], fa[C::TA];
#pragma unroll
      for (int i = 0; i < C::TW; ++i)
        fw[i] = *(const bf16x8*)(L + BM * C::BK + swz(wn * C::RW + i * 32 + (lane & 31), chunk));
#pragma unroll
      for (int j = 0; j < C::TA; ++j)
        fa[j] = *(const bf16x8*)(L + swz(wm * C::RA + j * 32 + (lane & 31), chunk));
#pragma unroll
      for (int i = 0; i < C::TW; ++i)
#pragma unroll
        for (int j = 0; j < C::TA; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fa[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store(cur ^ 1);
    __syncthreads();
  }

  const int col0 = ncol0 + wn * (EPI == EPI_SWIGLU ? C::RW / 2 : C::RW);
  store_tile<C::TW, C::TA, WDT, EPI>(a, ti, sg, acc, wm * C::RA, col0, lane);
}

// ============================================================== fp32 kernel
// 64 activation rows x 64 weight rows per block, BK = 16, 4x4 outputs per
// thread.  For SwiGLU the 64 weight rows are 32 W1 rows and the matching 32
// W3 rows, and a thread's 4 weight rows are {2c, 2c+1} of W1 and of W3.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a, int n_slots, int n_tiles) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int NCOL = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  int mt, nt;
  block_coords(real_mtiles(a, BM), n_tiles, mt, nt);
  if (mt < 0) return;
  TileInfo ti;
  Seg sg;
  if (!tile_info(a, mt, BM, ti, sg)) return;
  const int ncol0 = nt * NCOL;
  if (ncol0 >= sg.N) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int K = sg.K;
  const int kspan = K / a.ksplit, k_begin = blockIdx.y * kspan;
  const float* A = (const float*)sg.A;

  int wrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) wrow[q] = (EPI == EPI_SWIGLU) ? ((q < 2) ? 2 * tx + q : 32 + 2 * tx + q - 2) : 4 * tx + q;

  size_t arow[4];  // A row (element offset) of each staged row of this thread
#pragma unroll
  for (int q = 0; q < 4; ++q)
    arow[q] = (size_t)a_row(sg, ti.row0, min((tid + q * 256) >> 4, ti.nrows - 1)) * K;

  float acc[4][4] = {};
  for (int k0 = k_begin; k0 < k_begin + kspan; k0 += BK) {
    // stage: 64 rows x 16 k for A and B (4 elements per thread each)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + q * 256;
      const int r = idx >> 4, kk = idx & 15;
      As[kk][r] = A[arow[q] + k0 + kk];
      const float* base;
      int n;
      if (EPI == EPI_SWIGLU) {
        base = (const float*)((r < 32) ? sg.B0 : sg.B1);
        n = ncol0 + (r & 31);
      } else {
        base = (const float*)sg.B0;
        n = min(ncol0 + r, sg.N - 1);
      }
      Bs[kk][r] = base[(size_t)n * K + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(As[kk][ty * 4 + i], Bs[kk][wrow[q]], acc[i][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lrow = ty * 4 + i;
    if (lrow >= ti.nrows) continue;
    const size_t row = (size_t)(ti.row0 + lrow);
    float* Cr = (float*)sg.C + ((size_t)blockIdx.y * a.rows + row) * sg.N;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int q = 0; q < 2; ++q) Cr[ncol0 + 2 * tx + q] = silu(acc[i][q]) * acc[i][q + 2];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = ncol0 + 4 * tx + q;
        const bool bias = EPI == EPI_BIAS_F32 && a.bias && blockIdx.y == 0;
        if (n < sg.N) Cr[n] = acc[i][q] + (bias ? a.bias[n] : 0.f);
      }
    }
  }
}

// ============================================================== tile tables
// Inclusive prefix sum over the 512 threads of v, through LDS.
__device__ __forceinline__ int block_scan512(int* buf, int v) {
  const int e = threadIdx.x;
  buf[e] = v;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {
    const int u = (e >= off) ? buf[e - off] : 0;
    __syncthreads();
    buf[e] += u;
    __syncthreads();
  }
  const int r = buf[e];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(512) void tile_table_kernel(TileTableArgs t) {
  __shared__ int pre[512];
  __shared__ int tot[3];
  const int e = threadIdx.x;
  const int cnt = (e < t.E) ? t.offsets[e + 1] - t.offsets[e] : 0;
  for (int w = 0; w < 2; ++w) {
    const int bm = w == 0 ? t.bm0 : t.bm1;
    if (bm == 0) break;
    int32_t* table = w == 0 ? t.table0 : t.table1;
    const int n_slots = w == 0 ? t.n_slots0 : t.n_slots1;
    const int sh_tiles = (t.sh_rows + bm - 1) / bm;  // the extra segment E
    int total;
    if (bm == 256) {
      // Tiles by cost, so the launch ends on its cheapest tiles and the
      // XCDs are dealt tiles of like cost together: every expert's tiles
      // that run the full layout (more than 128 rows), then the extra
      // segment's, then the half-height last tiles (65-128 rows), then the
      // quarter-height ones (1-64 rows); experts in order within each class.
      // The split plan's K-pieces then come from the cheap tiles at the end.
      // Same box: Qwen-shaped fp8-weight layer gate-up -5.5%, down -8.1%;
      // DeepSeek-V3-shaped prefill gate-up -2.9%; Mixtral-shaped unchanged.
      const int rem = cnt % 256;
      const int nf = cnt / 256 + (rem > 128 ? 1 : 0);
      const int nh = (rem > 64 && rem <= 128) ? 1 : 0, nq = (rem > 0 && rem <= 64) ? 1 : 0;
      // one scan for both one-per-expert classes: each count is at most 512
      const int pf = block_scan512(pre, nf), phq = block_scan512(pre, nh | (nq << 16));
      const int ph = phq & 0xffff, pq = phq >> 16;
      if (e == 511) { tot[0] = pf; tot[1] = ph; tot[2] = pq; }
      __syncthreads();
      const int F = tot[0] + sh_tiles, H = tot[1], Q = tot[2];
      for (int i = 0; i < nf; ++i) table[pf - nf + i] = (e << kTableExpertShift) | i;
      for (int i = e; i < sh_tiles; i += 512) table[tot[0] + i] = (t.E << kTableExpertShift) | i;
      if (nh) table[F + ph - 1] = (e << kTableExpertShift) | (cnt / 256);
      if (nq) table[F + H + pq - 1] = (e << kTableExpertShift) | (cnt / 256);
      total = F + H + Q;
      __syncthreads();
    } else {
      const int tiles = (cnt + bm - 1) / bm;
      const int incl = block_scan512(pre, tiles);
      if (e == 511) tot[0] = incl;
      __syncthreads();
      for (int i = 0; i < tiles; ++i) table[incl - tiles + i] = (e << kTableExpertShift) | i;
      for (int i = e; i < sh_tiles; i += 512) table[tot[0] + i] = (t.E << kTableExpertShift) | i;
      total = tot[0] + sh_tiles;
      __syncthreads();
    }
    for (int s = total + e; s < n_slots; s += 512) table[s] = -1;
    if (e == 0) table[n_slots] = total;  // real m-tiles, read by every GEMM block
  }
}

template <int BM, int BN, int WDT, int EPI>
hipError_t launch_mfma(const GemmArgs& a, hipStream_t s) {
  using C = MfmaCfg<BM, BN, WDT, EPI>;
  const int n_slots = a.tile_table ? a.n_slots : (a.rows + BM - 1) / BM;
  const int n_tiles = (gemm_max_cols(a) + C::NCOL - 1) / C::NCOL;
  int nb = n_slots * n_tiles;
  nb = (nb + 7) & ~7;
  hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WDT, EPI>), dim3(nb, a.ksplit), dim3(C::NTHR), 0, s,
                     a, n_slots, n_tiles);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_f32(const GemmArgs& a, hipStream_t s) {
  const int ncol = (EPI == EPI_SWIGLU) ? 32 : 64;
  const int n_slots = a.tile_table ? a.n_slots : (a.rows + 63) / 64;
  const int n_tiles = (gemm_max_cols(a) + ncol - 1) / ncol;
  int nb = n_slots * n_tiles;
  nb = (nb + 7) & ~7;
  hipLaunchKernelGGL((gemm_f32_kernel<EPI>), dim3(nb, a.ksplit), dim3(256), 0, s, a, n_slots,
                     n_tiles);
  return hipGetLastError();
}

template <int WDT>
hipError_t launch_mfma_epi(const GemmArgs& a, hipStream_t s) {
  switch (a.epi) {
    case EPI_SWIGLU: return launch_mfma<128, 128, WDT, EPI_SWIGLU>(a, s);
    case EPI_STORE: return launch_mfma<128, 128, WDT, EPI_STORE>(a, s);
    default: return launch_mfma<128, 128, WDT, EPI_BIAS_F32>(a, s);
  }
}

// Row-major [mats][rows][cols] -> [mats][cols/32][rows][32], 16 bytes per
// thread in output order: a wave stores one contiguous kilobyte and loads
// runs of 32 * elem_bytes bytes from 32 / (2 / elem_bytes) rows.
__global__ __launch_bounds__(256) void pack_kblocked_kernel(const u32x4* __restrict__ src, int64_t mats, int rows,
                                                            int cols, int elem_bytes, u32x4* __restrict__ dst) {
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = 2 * elem_bytes;                   // 16-byte pieces of a plane row (32 elements)
  const size_t per_plane = (size_t)rows * per_row;
  const size_t per_mat = per_plane * (cols / 32);
  if (g >= per_mat * (size_t)mats) return;
  const size_t m = g / per_mat, in = g % per_mat;
  const int p = (int)(in / per_plane), rem = (int)(in % per_plane), r = rem / per_row, q = rem % per_row;
  const size_t row_pieces = (size_t)cols * elem_bytes / 16;  // 16-byte pieces of a source row
  dst[g] = src[m * rows * row_pieces + (size_t)r * row_pieces + (size_t)p * per_row + q];
}

}  // namespace

hipError_t launch_pack_kblocked(const void* src, int64_t mats, int rows, int cols, int elem_bytes, void* dst,
                                hipStream_t s) {
  const size_t pieces = (size_t)mats * rows * cols * elem_bytes / 16;
  if (pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kblocked_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s,
                     (const u32x4*)src, mats, rows, cols, elem_bytes, (u32x4*)dst);
  return hipGetLastError();
}

// Prefill-shaped problems with bf16 activations and bf16 or fp8 weights
// (enough rows per expert to fill 256-row tiles), and router logits of at
// least 1024 tokens, go to the direct-to-LDS 256-row kernel; the rest use
// 128-row tiles.
static bool use_big(const GemmArgs& a) {
  if (a.act == GD_FP8) return gemm_fp8_act_ok(a);
  if (a.act != GD_BF16 || a.wdt == GD_F32) return false;
  // router logits: worth a 256-wide tile only with at least 128 experts
  if (a.epi == EPI_BIAS_F32) return a.wdt == GD_BF16 && a.tile_table == nullptr && a.rows >= 1024 && a.N >= 128;
  const int segs = a.E > 0 ? a.E : 1;
  return a.rows >= 1024 && a.rows / segs >= 128;
}

// Decode-shaped grouped bf16 problems (on average at most one 32-row token
// block per expert) are weight streams: the weight-streaming kernel.
static bool use_decode(const GemmArgs& a) {
  if (a.act != GD_BF16 || a.wdt != GD_BF16 || a.epi == EPI_BIAS_F32) return false;
  if (a.offsets == nullptr || a.E <= 0) return false;
  return a.rows <= 32 * a.E;
}

// fp8 activations (the block-scaled dispatch payload) run only on the 256-row
// kernel's fp8 x fp8 gate-up path: the same shapes it takes with bf16
// activations, so the tile height matches the down projection's.
bool gemm_fp8_act_ok(const GemmArgs& a) {
  if (a.wdt != GD_FP8 || a.epi != EPI_SWIGLU || a.sh_rows > 0) return false;
  if (a.K % 64 != 0 || a.a_sstride % 16 != 0 || a.a_sstride * 32 < a.K) return false;
  const int segs = a.E > 0 ? a.E : 1;
  return a.rows >= 1024 && a.rows / segs >= 128;
}

int gemm_block_m(const GemmArgs& a) {
  if (a.act == GD_F32) return 64;
  return use_big(a) ? 256 : 128;
}

int gemm_max_slots(int rows, int E, int block_m, int sh_rows) {
  return (rows + block_m - 1) / block_m + E + (sh_rows + block_m - 1) / block_m;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  // K-blocked operands: bf16 A / the SwiGLU output, on the prefill kernel only
  // K-blocked routed weights: bf16 / fp8 expert GEMMs (never the router's)
  if (a.b_blk && (a.act == GD_F32 || a.wdt == GD_F32 || a.epi == EPI_BIAS_F32 || a.ksplit > 1))
    return hipErrorInvalidValue;
  if ((a.a_blk || a.sh_a_blk || a.c_blk) &&
      !(a.act != GD_F32 && !use_decode(a) && use_big(a) && a.epi != EPI_BIAS_F32 &&
        (!a.c_blk || a.epi == EPI_SWIGLU) && (!a.a_blk || a.act == GD_BF16) &&
        (!a.sh_a_blk || a.act == GD_BF16)))
    return hipErrorInvalidValue;
  // 64-column planes: the SwiGLU GEMM, K (and the extra segment's K) a
  // multiple of 64
  if (a.a_blk < 0 || a.a_blk > 2 || a.sh_a_blk < 0 || a.sh_a_blk > 2 ||
      ((a.a_blk == 2 || a.sh_a_blk == 2) &&
       (a.epi != EPI_SWIGLU || a.K % 64 != 0 || (a.sh_rows > 0 && a.shK % 64 != 0))))
    return hipErrorInvalidValue;
  if (a.act == GD_F32) {
    switch (a.epi) {
      case EPI_SWIGLU: return launch_f32<EPI_SWIGLU>(a, s);
      case EPI_STORE: return launch_f32<EPI_STORE>(a, s);
      default: return launch_f32<EPI_BIAS_F32>(a, s);
    }
  }
  if (a.act == GD_FP8 && (!gemm_fp8_act_ok(a) || a.a_scales == nullptr)) return hipErrorInvalidValue;
  if (use_decode(a)) return launch_gemm_decode(a, s);
  if (use_big(a)) return launch_gemm_big(a, s);
  return a.wdt == GD_FP8 ? launch_mfma_epi<GD_FP8>(a, s) : launch_mfma_epi<GD_BF16>(a, s);
}

hipError_t launch_tile_tables(const TileTableArgs& t, hipStream_t s) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(512), 0, s, t);
  return hipGetLastError();
}

}  // namespace moe
