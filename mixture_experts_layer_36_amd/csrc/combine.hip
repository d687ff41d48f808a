// Combine: each token's k expert rows, weighted by its gates, summed in fp32
// back in token order (plus the shared expert's row), then stored in the
// activation dtype.
//
// The weighted sum of the expert outputs is the combine step of "Tensor vs
// Expert vs Data Parallelism for MoE Serving" (section "Deeper Analysis:
// Communication, Overlap and Load Balance", Figure 2) and of "Expert-Parallel
// MoE Inference: Serving Sparse Models at Scale" (section "Deeper Analysis",
// Figure 2).  No atomics: a token gathers its own k rows through inv_pos, so
// the result is deterministic.  The sum runs j = 0..k-1, then the shared row;
// an assignment dropped for capacity (inv_pos = -1) contributes nothing.
// One block per token row, a thread per 16-byte chunk of the row: one pass
// of loads and stores (896 threads for d = 7168, 512 for d = 4096).  Against
// 256-thread blocks (3.5 passes at d = 7168, the last one half idle) and
// two-pass blocks, the DeepSeek-V3-shaped prefill combine went 430 -> 421 ->
// 400 us and the Qwen-shaped one 108 -> 104 us.  HBM-bound; a thread has its
// k row loads in flight together.  The expert rows are read once and
// the output written once, so both go non-temporal (kept out of the caches
// the next layer's data would use): DeepSeek-V3-shaped prefill combine
// 473 -> 411 us, Qwen-shaped 123 -> 99 us.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kMaxK = 16;

// KM >= k bounds the token's rows at compile time, so all k row loads (and
// the shared row's) are issued before the first is consumed: one 16-byte
// load per row in flight per thread rather than one in all.
template <int KM>
__global__ __launch_bounds__(1024) void combine_bf16_kernel(CombineArgs a) {
  __shared__ int s_row[kMaxK];
  __shared__ float s_g[kMaxK];
  const int t = blockIdx.x;
  if (threadIdx.x < a.k) {
    s_row[threadIdx.x] = a.inv_pos[(size_t)t * a.k + threadIdx.x];
    s_g[threadIdx.x] = a.topk_w[(size_t)t * a.k + threadIdx.x];
  }
  __syncthreads();
  int row[KM];
  float g[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    row[j] = j < a.k ? s_row[j] : -1;  // -1: no row (past k, or dropped for capacity)
    g[j] = j < a.k ? s_g[j] : 0.f;
  }
  const int nvec = a.d / 8;  // 8 bf16 per 16 bytes
  const u32x4* __restrict__ y = (const u32x4*)a.y_perm;
  const u32x4* __restrict__ ys = (const u32x4*)a.shared_y;
  u32x4* __restrict__ out = (u32x4*)a.out;
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    u32x4 r[KM], rs = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < KM; ++j) r[j] = row[j] >= 0 ? __builtin_nontemporal_load(&y[(size_t)row[j] * nvec + v]) : rs;
    if (ys) rs = __builtin_nontemporal_load(&ys[(size_t)t * nvec + v]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (row[j] < 0) continue;  // no contribution
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += g[j] * bf16_to_f32(r[j][q] & 0xffffu);
        acc[2 * q + 1] += g[j] * bf16_to_f32(r[j][q] >> 16);
      }
    }
    if (ys) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(rs[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(rs[q] >> 16);
      }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    __builtin_nontemporal_store(o, &out[(size_t)t * nvec + v]);
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(CombineArgs a) {
  __shared__ int s_row[kMaxK];
  __shared__ float s_g[kMaxK];
  const int t = blockIdx.x;
  if (threadIdx.x < a.k) {
    s_row[threadIdx.x] = a.inv_pos[(size_t)t * a.k + threadIdx.x];
    s_g[threadIdx.x] = a.topk_w[(size_t)t * a.k + threadIdx.x];
  }
  __syncthreads();
  const int nvec = a.d / 4;
  const f32x4* y = (const f32x4*)a.y_perm;
  const f32x4* ys = (const f32x4*)a.shared_y;
  f32x4* out = (f32x4*)a.out;
  for (int v = threadIdx.x; v < nvec; v += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.k; ++j) {
      if (s_row[j] < 0) continue;  // dropped for capacity: no contribution
      const f32x4 r = y[(size_t)s_row[j] * nvec + v];
      const float g = s_g[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += g * r[q];
    }
    if (ys) {
      const f32x4 r = ys[(size_t)t * nvec + v];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += r[q];
    }
    out[(size_t)t * nvec + v] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  // bf16: a thread per 16-byte chunk of the row (more passes past 1024),
  // whole wavefronts, at least 64 threads (the first k threads stage the
  // token's rows and gates)
  const int nvec = a.d / 8;
  int thr = (nvec + 63) / 64 * 64;
  thr = thr < 64 ? 64 : thr > 1024 ? 1024 : thr;
  if (a.act != GD_BF16)
    hipLaunchKernelGGL(combine_f32_kernel, dim3(a.T), dim3(256), 0, s, a);
  else if (a.k <= 2)
    hipLaunchKernelGGL(combine_bf16_kernel<2>, dim3(a.T), dim3(thr), 0, s, a);
  else if (a.k <= 4)
    hipLaunchKernelGGL(combine_bf16_kernel<4>, dim3(a.T), dim3(thr), 0, s, a);
  else if (a.k <= 8)
    hipLaunchKernelGGL(combine_bf16_kernel<8>, dim3(a.T), dim3(thr), 0, s, a);
  else
    hipLaunchKernelGGL(combine_bf16_kernel<kMaxK>, dim3(a.T), dim3(thr), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
