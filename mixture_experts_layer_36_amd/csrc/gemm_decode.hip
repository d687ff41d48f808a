// Decode-shaped grouped GEMM: few rows per expert, so the layer is a stream of
// expert weights ("read the whole expert weight matrix to do almost no work",
// "Tensor vs Expert vs Data Parallelism for MoE Serving", section "Why
// sparsity demands a large batch").  The kernel is built to keep HBM busy:
//   * one block per (segment, slice of 128 weight rows): 4 wavefronts, each
//     owning 32 weight rows x a block of 32 token rows -- one
//     v_mfma_f32_32x32x16_bf16 per k16 step, weights as the MFMA row operand;
//     the down projection takes kStoreSlices slices per block, and a segment
//     of one token block runs their stages through the ring back to back;
//   * weights and token rows go global -> LDS with buffer_load_dwordx4 ... lds
//     (128-byte row segments, fully coalesced; weights non-temporal, read
//     once) through a 4-deep ring of 20 KB
//     stages refilled four stages ahead, so two blocks per CU keep ~160 KB of
//     loads in flight; fragment reads use the (r ^ (r >> 3)) & 7 chunk
//     swizzle of 128-byte rows, measured conflict-free on gfx950;
//   * SwiGLU: waves 0-1 hold u (W1 rows), waves 2-3 the matching v (W3 rows);
//     v crosses through LDS in the epilogue;
//   * a segment with more than 32 rows loops over token blocks (weights are
//     re-read from L2/MALL); rows past a segment's end read as zero through
//     the buffer descriptor and are never stored.
// Segments are the routed experts (rows [offsets[e], offsets[e+1]) of the
// expert-contiguous buffer) plus, optionally, segment E: the shared expert
// over all tokens in order.
#include "gemm_common.hpp"

namespace moe {
namespace {

constexpr int WR = 128;        // weight rows per block
constexpr int TB = 32;         // token rows per token block
constexpr int BK = 64;         // k per stage (128-byte rows)
[[maybe_unused]] constexpr int STAGES = 4;
constexpr int NTHR = 256;
constexpr int W_ELEMS = WR * BK;
constexpr int T_ELEMS = TB * BK;
[[maybe_unused]] constexpr int STAGE = W_ELEMS + T_ELEMS;     // bf16 elements per stage (20 KB)
[[maybe_unused]] constexpr int W_LOADS = W_ELEMS / 8 / NTHR;  // 16-byte loads per thread per stage: 4
[[maybe_unused]] constexpr int T_LOADS = T_ELEMS / 8 / 64;    // token loads, issued by wave 0 only: 4
[[maybe_unused]] constexpr int kBufferFlags = 0x00020000;
// Cache policy of the weight loads: non-temporal (the nt bit).  A block
// streams its weight rows once; the hint raised a streaming read on MI355X
// from 6.26 to 7.09 TB/s, and the DeepSeek-V3-shaped decode gate-up GEMM
// from 2549 to 2356 us (token rows, re-read by every slice, stay cached).
[[maybe_unused]] constexpr int kWeightPolicy = 2;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

[[maybe_unused]] __device__ __forceinline__ int dswz(int r) { return (r ^ (r >> 3)) & 7; }
[[maybe_unused]] __device__ __forceinline__ int doff(int r, int c) {
  return r * BK + ((c ^ dswz(r)) << 3);
}
template <int N>
__device__ __forceinline__ void dwait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
[[maybe_unused]] __device__ __forceinline__ void dbarrier() { asm volatile("s_barrier" ::: "memory"); }

// Slices per block of the down projection (EPI_STORE): four slices' stages
// run through one ring (DeepSeek-V3-shaped decode down GEMM 1268 -> 1228 us;
// 2 slices: 1250 us; 7 or more: slower, the blocks then too long for the
// launch's tail).  SwiGLU keeps one slice per block: its epilogue exchanges
// v through the stage buffers.
constexpr int kStoreSlices = 4;
template <int EPI, int SPB>
__global__ __launch_bounds__(NTHR, 2) void gemm_decode_kernel(GemmArgs a, int n_slices) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) __bf16 lds[STAGES * STAGE];
  // the shared segment (all T rows, several token blocks) is dispatched
  // first, one slice per block, so that its longer blocks neither end up in
  // the tail of the launch nor grow into its critical path; then the routed
  // segments, SPB slices per block
  const int has_sh = a.sh_rows > 0 ? 1 : 0;
  const int n_groups = (n_slices + SPB - 1) / SPB;
  const int sh_blocks = has_sh ? n_slices : 0;
  int seg, first, per;
  if ((int)blockIdx.x < sh_blocks) {
    seg = a.E;
    first = blockIdx.x;
    per = 1;
  } else {
    const int b = blockIdx.x - sh_blocks;
    seg = b / n_groups;
    if (seg >= a.E) return;
    first = (b % n_groups) * SPB;
    per = SPB;
  }

  // segment operands
  const bool shared = seg == a.E;
  int row0, nrows;
  const int32_t* amap = nullptr;  // routed rows through the row map (fused dispatch gather)
  const char *A, *B0, *B1;
  char* Cp;
  int N, K;
  bool wblk = false;  // weights K-blocked (routed experts only)
  if (shared) {
    row0 = 0;
    nrows = a.sh_rows;
    A = (const char*)a.shA;
    B0 = (const char*)a.shB0;
    B1 = (const char*)a.shB1;
    Cp = (char*)a.shC;
    N = a.shN;
    K = a.shK;
  } else {
    row0 = a.offsets[seg];
    nrows = a.offsets[seg + 1] - row0;
    const size_t woff = (size_t)seg * a.N * a.K * 2;
    A = (const char*)a.A;
    amap = a.a_map;
    B0 = (const char*)a.B0 + woff;
    B1 = a.B1 ? (const char*)a.B1 + woff : nullptr;
    Cp = (char*)a.C;
    N = a.N;
    K = a.K;
    wblk = a.b_blk != 0;
  }
  const int ncol = (EPI == EPI_SWIGLU) ? WR / 2 : WR;  // output columns per slice
  if (nrows <= 0) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KT = K / BK;
  // the slices of this block: first .. first + nsl - 1 (those inside N)
  const int nsl = min(per, (N + ncol - 1) / ncol - first);
  if (nsl <= 0) return;

  // weight rows of this slice: SwiGLU = 64 W1 rows then the same 64 W3 rows.
  // K-blocked weights: the descriptor starts at the slice's first row in
  // plane 0 and spans the rest of the matrix; a 64-k stage covers two
  // 32-column planes of N rows x 64 bytes.
  const int wrows = (EPI == EPI_SWIGLU) ? WR / 2 : WR;
  const int wplane = wblk ? N * 64 : 0;
  const int wstep = wblk ? 2 * wplane : BK * 2;  // bytes from one stage's slice to the next
  // a slice's weight descriptor (SGPRs): from its first row to the end of
  // the matrix's span for it
  auto wrsrc = [&](const char* B, int slice) {
    const int c0 = slice * ncol;
    const size_t wstart = (size_t)c0 * (wblk ? 64 : K * 2);
    const int wbytes = wblk ? (K / 32) * wplane - c0 * 64 : wrows * K * 2;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(B + wstart), (short)0, wbytes, kBufferFlags);
  };
  // slot s of a load instruction's 64 slots: row s / 8, physical chunk s % 8
  // holding logical chunk (s % 8) ^ dswz(row)
  uint32_t w_off[W_LOADS];
  bool w_is1[W_LOADS];
#pragma unroll
  for (int j = 0; j < W_LOADS; ++j) {
    const int s = (wave * W_LOADS + j) * 64 + lane;
    const int r = s >> 3, c = (s & 7) ^ dswz(r);
    w_is1[j] = (EPI == EPI_SWIGLU) && ((wave * W_LOADS + j) * 8 >= WR / 2);  // uniform per load
    const int n = (EPI == EPI_SWIGLU) ? (r % (WR / 2)) : r;
    w_off[j] = wblk ? (uint32_t)((c >> 2) * wplane + n * 64 + (c & 3) * 16) : (uint32_t)(n * K + c * 8) * 2u;
  }
  const int tr = lane >> 3;  // token rows lane/8 + 8 j
  const int tc = (lane & 7);

  f32x16 acc;
  if (EPI == EPI_STORE && nsl > 1 && nrows <= TB) {
    // One token block, several slices: one ring runs through the slices'
    // stages back to back, so the next slice's first stages are in flight
    // while this one's results are stored (from registers; LDS untouched).
    const uint32_t t_bytes = (uint32_t)(amap ? a.a_map_rows : nrows) * K * 2;
    const __amdgpu_buffer_rsrc_t tok = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(amap ? A : A + (size_t)row0 * K * 2), (short)0, t_bytes, kBufferFlags);
    uint32_t t_off[T_LOADS];
#pragma unroll
    for (int j = 0; j < T_LOADS; ++j) {
      const int r = tr + 8 * j, c = tc ^ dswz(r);
      const int ar = amap ? (r < nrows ? amap[row0 + r] : -1) : r;
      t_off[j] = ar < 0 ? t_bytes : (uint32_t)(ar * K + c * 8) * 2u;
    }
    int isl = 0, ikt = 0;  // the next stage to issue: slice, k-stage
    auto issue_next = [&](int buf) {
      const bool past = isl >= nsl;  // past the end: re-load the last stage into a buffer never read
      const int sl = past ? nsl - 1 : isl, kt = past ? KT - 1 : ikt;
      const __amdgpu_buffer_rsrc_t w = wrsrc(B0, first + sl);
      __bf16* st = lds + buf * STAGE;
#pragma unroll
      for (int j = 0; j < W_LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w, (lds_ptr_t)(st + (wave * W_LOADS + j) * 512), 16, w_off[j],
                                                 kt * wstep, 0, kWeightPolicy);
      if (wave == 0) {
#pragma unroll
        for (int j = 0; j < T_LOADS; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(tok, (lds_ptr_t)(st + W_ELEMS + j * 512), 16, t_off[j],
                                                   kt * BK * 2, 0, 0);
      }
      if (!past && ++ikt == KT) {
        ikt = 0;
        ++isl;
      }
    };
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll
    for (int s = 0; s < STAGES; ++s) issue_next(s);
    const int t = lane & 31;
    int ckt = 0, csl = 0;
    for (int g = 0; g < nsl * KT; ++g) {
      if (wave == 0) dwait_vmcnt<3 * (W_LOADS + T_LOADS)>();
      else dwait_vmcnt<3 * W_LOADS>();
      dbarrier();
      const __bf16* L = lds + (g % STAGES) * STAGE;
      bf16x8 fw[BK / 16], ft[BK / 16];
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int c = kk * 2 + (lane >> 5);
        fw[kk] = *(const bf16x8*)(L + doff(wave * 32 + (lane & 31), c));
        ft[kk] = *(const bf16x8*)(L + W_ELEMS + doff(lane & 31, c));
      }
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[kk], ft[kk], acc, 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of the stage done
      dbarrier();
      issue_next(g % STAGES);
      if (++ckt == KT) {  // slice first + csl complete
        if (t < nrows) {
          const size_t row = (size_t)(row0 + t);
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int n = (first + csl) * ncol + wave * 32 + gq * 8 + (lane >> 5) * 4;
            u32x2 o;
            o[0] = pack_bf16x2(acc[gq * 4 + 0], acc[gq * 4 + 1]);
            o[1] = pack_bf16x2(acc[gq * 4 + 2], acc[gq * 4 + 3]);
            *(u32x2*)((uint16_t*)Cp + row * N + n) = o;
          }
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[q] = 0.f;
        ckt = 0;
        ++csl;
      }
    }
    dwait_vmcnt<0>();  // the re-loads past the end land before the block can exit
    return;
  }
  for (int sli = 0; sli < nsl; ++sli) {
    const int ncol0 = (first + sli) * ncol;
    const __amdgpu_buffer_rsrc_t w0 = wrsrc(B0, first + sli);
    const __amdgpu_buffer_rsrc_t w1 = wrsrc(EPI == EPI_SWIGLU ? B1 : B0, first + sli);
    for (int tb0 = 0; tb0 < nrows; tb0 += TB) {
      const int tb_rows = min(TB, nrows - tb0);
      // rows past the block's end read as zero: offset beyond the descriptor
      const uint32_t t_bytes = (uint32_t)(amap ? a.a_map_rows : tb_rows) * K * 2;
      const __amdgpu_buffer_rsrc_t tok = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(amap ? A : A + (size_t)(row0 + tb0) * K * 2), (short)0, t_bytes, kBufferFlags);
      uint32_t t_off[T_LOADS];
#pragma unroll
      for (int j = 0; j < T_LOADS; ++j) {
        const int r = tr + 8 * j, c = tc ^ dswz(r);
        const int ar = amap ? (r < tb_rows ? amap[row0 + tb0 + r] : -1) : r;
        t_off[j] = ar < 0 ? t_bytes : (uint32_t)(ar * K + c * 8) * 2u;
      }
      auto issue = [&](int kt, int buf) {
        __bf16* st = lds + buf * STAGE;
        const int kb = min(kt, KT - 1) * BK * 2;
        const int wk = min(kt, KT - 1) * wstep;
#pragma unroll
        for (int j = 0; j < W_LOADS; ++j) {
          const lds_ptr_t dst = (lds_ptr_t)(st + (wave * W_LOADS + j) * 512);
          if (w_is1[j])
            __builtin_amdgcn_raw_ptr_buffer_load_lds(w1, dst, 16, w_off[j], wk, 0, kWeightPolicy);
          else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(w0, dst, 16, w_off[j], wk, 0, kWeightPolicy);
        }
        if (wave == 0) {
#pragma unroll
          for (int j = 0; j < T_LOADS; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(tok, (lds_ptr_t)(st + W_ELEMS + j * 512), 16,
                                                     t_off[j], kb, 0, 0);
        }
      };
      // wave 0 issues W_LOADS + T_LOADS loads per stage, the others W_LOADS
      auto wait_stage = [&](int stages_after) {
        if (wave == 0) {
          if (stages_after >= 3) dwait_vmcnt<3 * (W_LOADS + T_LOADS)>();
          else if (stages_after == 2) dwait_vmcnt<2 * (W_LOADS + T_LOADS)>();
          else if (stages_after == 1) dwait_vmcnt<W_LOADS + T_LOADS>();
          else dwait_vmcnt<0>();
        } else {
          if (stages_after >= 3) dwait_vmcnt<3 * W_LOADS>();
          else if (stages_after == 2) dwait_vmcnt<2 * W_LOADS>();
          else if (stages_after == 1) dwait_vmcnt<W_LOADS>();
          else dwait_vmcnt<0>();
        }
      };

#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll
      for (int s = 0; s < STAGES; ++s) issue(s, s);
      for (int kt = 0; kt < KT; ++kt) {
        // stage kt resident for everyone; stage kt-1 (same buffer as kt+3) retired
        wait_stage(STAGES - 1);
        dbarrier();
        const __bf16* L = lds + (kt % STAGES) * STAGE;
        bf16x8 fw[BK / 16], ft[BK / 16];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const int c = kk * 2 + (lane >> 5);
          fw[kk] = *(const bf16x8*)(L + doff(wave * 32 + (lane & 31), c));
          ft[kk] = *(const bf16x8*)(L + W_ELEMS + doff(lane & 31, c));
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[kk], ft[kk], acc, 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage kt done
        dbarrier();
        issue(kt + STAGES, kt % STAGES);
      }
      wait_stage(0);  // drain the stages issued past the end before the buffers are reused
      dbarrier();

      // ---- epilogue: lane holds weight rows g*8 + (lane/32)*4 + q of this
      // wave's 32 for token (lane % 32)
      const int t = lane & 31;
      const bool valid = t < tb_rows;
      const size_t row = (size_t)(row0 + tb0 + t);
      if (EPI == EPI_SWIGLU) {
        float* xch = (float*)lds;  // v from waves 2-3 -> waves 0-1 (stage buffers are idle)
        if (wave >= 2) {
#pragma unroll
          for (int q = 0; q < 16; ++q) xch[((wave - 2) * 16 + q) * 64 + lane] = acc[q];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        dbarrier();
        if (wave < 2 && valid) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = ncol0 + wave * 32 + g * 8 + (lane >> 5) * 4;
            float hv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float v = xch[(wave * 16 + g * 4 + q) * 64 + lane];
              hv[q] = silu(acc[g * 4 + q]) * v;
            }
            u32x2 o;
            o[0] = pack_bf16x2(hv[0], hv[1]);
            o[1] = pack_bf16x2(hv[2], hv[3]);
            *(u32x2*)((uint16_t*)Cp + row * N + n) = o;
          }
        }
        dbarrier();  // exchange buffer free before the next token block's loads
      } else if (valid) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = ncol0 + wave * 32 + g * 8 + (lane >> 5) * 4;
          u32x2 o;
          o[0] = pack_bf16x2(acc[g * 4 + 0], acc[g * 4 + 1]);
          o[1] = pack_bf16x2(acc[g * 4 + 2], acc[g * 4 + 3]);
          *(u32x2*)((uint16_t*)Cp + row * N + n) = o;
        }
      }
    }
  }
#endif
}

}  // namespace

hipError_t launch_gemm_decode(const GemmArgs& a, hipStream_t s) {
  const int ncol = (a.epi == EPI_SWIGLU) ? WR / 2 : WR;
  const int n_slices = (gemm_max_cols(a) + ncol - 1) / ncol;
  const int n_seg = a.E + (a.sh_rows > 0 ? 1 : 0);
  if (a.epi == EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_decode_kernel<EPI_SWIGLU, 1>), dim3(n_seg * n_slices), dim3(NTHR), 0, s, a, n_slices);
  else
    hipLaunchKernelGGL((gemm_decode_kernel<EPI_STORE, kStoreSlices>),
                       dim3((a.sh_rows > 0 ? n_slices : 0) + a.E * ((n_slices + kStoreSlices - 1) / kStoreSlices)),
                       dim3(NTHR), 0, s, a, n_slices);
  return hipGetLastError();
}

}  // namespace moe
