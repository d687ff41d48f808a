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
//   * LDS rows of BK elements with 16-byte chunks XOR-swizzled by row
//     ((r >> 2) & 3 for 64-byte rows, (r ^ (r >> 3)) & 7 for 128-byte rows):
//     measured on gfx950 (64 banks; a 128-bit read is served 16 lanes at a
//     time), these make the fragment reads of 32 rows x 1 chunk
//     conflict-free.  A direct load writes 64 consecutive 16-byte slots, so
//     each lane fetches the global chunk that belongs in its slot.
#include "gemm_common.hpp"

namespace moe {
namespace {

#ifndef MOE_BIG_WN
#define MOE_BIG_WN 2
#endif
constexpr int BM = 256, BK = 32, STAGES = 4;
constexpr int CH = BK / 8;        // 16-byte chunks per LDS row
[[maybe_unused]] constexpr int KK = BK / 16;       // k16 MFMA steps per stage

// WN wavefronts along the weight rows, 2 along the activation rows.
template <int BN, int WN>
struct BigCfg {
  static constexpr int NTHR = 128 * WN;
  static constexpr int RA = BM / 2;   // activation rows per wave
  static constexpr int RW = BN / WN;  // weight rows per wave
  static constexpr int TA = RA / 32;
  static constexpr int TW = RW / 32;
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int B_ELEMS = BN * BK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;          // bf16 elements per stage
  static_assert(STAGES * STAGE * 2 <= 160 * 1024, "LDS");
  static constexpr int A_LOADS = BM * BK / 8 / NTHR;       // 16-byte loads per thread
  static constexpr int B_LOADS = BN * BK / 8 / NTHR;
  static constexpr int LOADS = A_LOADS + B_LOADS;
};

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

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Buffer descriptor word 3 for raw 32-bit-format buffers on gfx9-family GPUs.
[[maybe_unused]] constexpr int kBufferFlags = 0x00020000;

template <int BN, int WN, int EPI>
__global__ __launch_bounds__(128 * WN, 1) void gemm_big_kernel(GemmArgs a, int n_slots,
                                                                          int n_tiles) {
  // device pass only: the host pass needs just the launch stub
#if defined(__HIP_DEVICE_COMPILE__)
  using C = BigCfg<BN, WN>;
  __shared__ __attribute__((aligned(1024))) __bf16 lds[STAGES * C::STAGE];

  int mt, nt;
  block_coords(real_mtiles(a, BM), n_tiles, mt, nt);
  if (mt < 0) return;
  TileInfo ti;
  Seg sg;
  if (!tile_info(a, mt, BM, ti, sg)) return;
  const int ncol0 = nt * (EPI == EPI_SWIGLU ? BN / 2 : BN);
  if (ncol0 >= sg.N) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: SGPR arithmetic
  const int wm = wave / WN, wn = wave % WN;
  const int K = sg.K;

  // Direct loads go through buffer resources: a block-uniform descriptor
  // (SGPRs) per operand, a 32-bit per-lane byte offset fixed across stages
  // and the stage's k offset as the scalar offset, so each load is a single
  // buffer_load_dwordx4 ... lds with no per-stage address arithmetic.  The
  // descriptor's size bounds every access to the tile's own rows.  Slot s of
  // a stage's tile is row s / CH, physical chunk s % CH, which holds logical
  // chunk (s % CH) ^ swz(row).
  const int KT = K / BK;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sg.A + (size_t)ti.row0 * K * 2), (short)0, ti.nrows * K * 2, kBufferFlags);
  uint32_t a_off[C::A_LOADS];
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int s = (wave * C::A_LOADS + j) * 64 + lane;
    const int r = s / CH, c = (s % CH) ^ swz(r);
    const int rr = min(r, ti.nrows - 1);
    a_off[j] = (uint32_t)(rr * K + c * 8) * 2u;
  }
  // B: SwiGLU tiles take each wave's RW rows as RW/2 rows of W1 then the same
  // columns of W3 (one descriptor each); the 64 slots of one load are 64/CH
  // consecutive rows inside one half, so the choice is uniform per load.
  const int b_rows = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const size_t b_start = (size_t)ncol0 * K * 2;
  const __amdgpu_buffer_rsrc_t b0_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sg.B0 + b_start), (short)0, b_rows * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t b1_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((EPI == EPI_SWIGLU ? sg.B1 : sg.B0) + b_start), (short)0, b_rows * K * 2, kBufferFlags);
  uint32_t b_off[C::B_LOADS];
  bool b_w3[C::B_LOADS];
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int s = (wave * C::B_LOADS + j) * 64 + lane;
    const int r = s / CH, c = (s % CH) ^ swz(r);
    int n = r;  // row offset from ncol0
    b_w3[j] = false;
    if (EPI == EPI_SWIGLU) {
      const int half = C::RW / 2;
      const int r0 = (wave * C::B_LOADS + j) * 64 / CH;
      b_w3[j] = (r0 % C::RW) >= half;
      n = (r / C::RW) * half + (r % C::RW) % half;
    }
    b_off[j] = (uint32_t)(n * K + c * 8) * 2u;
  }

  // Stages past the end re-load the last stage into a buffer that is never
  // read again: every iteration then issues the same loads, the vmcnt waits
  // are constants and the refill can be scheduled between the MFMAs.
  // part 0 = the A loads of a stage, part 1 = its B loads
  auto issue_part = [&](int kt, int buf, int part) {
    __bf16* st = lds + buf * C::STAGE;
    const int kb = min(kt, KT - 1) * BK * 2;  // byte offset of the stage's k-slice
    if (part == 0) {
#pragma unroll
      for (int j = 0; j < C::A_LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (lds_ptr_t)(st + (wave * C::A_LOADS + j) * 512), 16, a_off[j], kb, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < C::B_LOADS; ++j) {
        const lds_ptr_t dst = (lds_ptr_t)(st + C::A_ELEMS + (wave * C::B_LOADS + j) * 512);
        if (b_w3[j])
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b1_rsrc, dst, 16, b_off[j], kb, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b0_rsrc, dst, 16, b_off[j], kb, 0, 0);
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
  struct Frags {
    bf16x8 w[C::TW], x[C::TA];
  };
  auto read_frags = [&](Frags& F, const __bf16* L, int kk) {
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::TW; ++i)
      F.w[i] = *(const bf16x8*)(L + C::A_ELEMS + lds_off(wn * C::RW + i * 32 + (lane & 31), c));
#pragma unroll
    for (int j = 0; j < C::TA; ++j)
      F.x[j] = *(const bf16x8*)(L + lds_off(wm * C::RA + j * 32 + (lane & 31), c));
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
  wait_vmcnt<2 * C::LOADS + C::A_LOADS>();  // stage 0 done
  barrier_only();

  Frags F[2];
  read_frags(F[0], lds, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const __bf16* L = lds + (kt % STAGES) * C::STAGE;
    // step 0: next fragments of this stage, B half of stage kt+3
    read_frags(F[1], L, 1);
    issue_part(kt + 3, (kt + 3) % STAGES, 1);
    mfmas(F[0]);
    interleave_refill();
    // step 1: stage kt+1 resident and stage kt retired everywhere, then the
    // A half of stage kt+4 into buffer kt % 4 and stage kt+1's first fragments
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    wait_vmcnt<2 * C::LOADS>();
    barrier_only();
    issue_part(kt + 4, kt % STAGES, 0);
    read_frags(F[0], lds + ((kt + 1) % STAGES) * C::STAGE, 0);
    mfmas(F[1]);
    interleave_refill();
  }

  const int col0 = ncol0 + wn * (EPI == EPI_SWIGLU ? C::RW / 2 : C::RW);
  store_tile<C::TW, C::TA, GD_BF16, EPI>(a, ti, sg, acc, wm * C::RA, col0, lane);
#endif
}

template <int BN, int EPI, int WN = MOE_BIG_WN>
hipError_t launch_big(const GemmArgs& a, hipStream_t s) {
  const int n_slots = a.tile_table ? a.n_slots : (a.rows + BM - 1) / BM;
  const int ncol = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int n_tiles = gemm_max_cols(a) / ncol;
  int nb = n_slots * n_tiles;
  nb = (nb + 7) & ~7;
  hipLaunchKernelGGL((gemm_big_kernel<BN, WN, EPI>), dim3(nb), dim3(BigCfg<BN, WN>::NTHR), 0, s, a,
                     n_slots, n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_big(const GemmArgs& a, hipStream_t s) {
  if (a.epi == EPI_SWIGLU) return launch_big<256, EPI_SWIGLU>(a, s);
  return (a.N % 256 == 0) ? launch_big<256, EPI_STORE>(a, s) : launch_big<128, EPI_STORE>(a, s);
}

}  // namespace moe
