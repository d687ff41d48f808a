// Router selection: scores, optional group limit, top-k and gates, one
// wavefront per token.
//
// The logits z = x Wr^T + b come from the grouped-GEMM kernel (EPI_BIAS_F32)
// as split-K partial sums, added here in a fixed order so the result is
// deterministic and identical router rows give identical logits.
// Following the per-token routing path of "Expert-Parallel MoE Inference:
// Serving Sparse Models at Scale" (section "Deeper Analysis", first paragraph,
// Figure 2): scores are softmax over the E logits or the element-wise sigmoid,
// the k best eligible experts are kept, and their gates are the scores,
// optionally divided by their sum over the chosen k.
//
// Selection compares packed 64-bit keys (order-preserving bits of the fp32
// logit << 32 | ~expert id), so the largest key is the largest score with ties
// going to the lower id.  Softmax and sigmoid are strictly increasing in the
// logit, so ranking logits ranks scores.  Each lane holds experts
// lane, lane+64, ... (up to 8 for E <= 512); the wave-wide maximum uses DPP
// moves within rows of 16 lanes and one read lane per row.  With a group limit (the single-GPU
// form of node-limited routing, same page, section "Load imbalance and how to
// fight it"), group scores (sum of each contiguous group's two largest scores)
// are ranked and groups outside the best topk_group are masked out: in
// registers (shuffles) when the groups tile the 64-expert columns, else
// through LDS.  Batching the partial-sum loads and ranking the groups in
// registers took the DeepSeek-V3-shaped prefill route stage from 146 to
// 141 us and the Qwen-shaped one from 61 to 54 us.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxE = 512;
constexpr int kMaxGroups = 64;

__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// 64-bit lane move through DPP (VALU data-parallel primitives, no LDS trip).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
// Wave-wide maximum, the same in every lane: within each row of 16 lanes by
// DPP swaps (quad_perm [1,0,3,2], [2,3,0,1]) and rotations (row_ror 4, 8),
// then across the four rows from one lane of each.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x124>(v));  // row_ror 4
  v = max_u64(v, dpp_u64<0x128>(v));  // row_ror 8
  return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)),
                 max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// NV = ceil(E / 64) expert columns per lane.
template <int NV>
__global__ __launch_bounds__(kWaves * 64) void route_select_kernel(RouteSelectArgs a) {
  __shared__ float s_score[kWaves][kMaxE];
  __shared__ float s_gscore[kWaves][kMaxGroups];
  __shared__ int s_keep[kWaves][kMaxGroups];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kWaves + wave;
  const bool live = t < a.T;                 // whole-wave condition
  const int tt = live ? t : a.T - 1;         // dead waves still reach every barrier
  const float* zrow = a.z + (size_t)tt * a.E;
  const size_t zsplit = (size_t)a.T * a.E;  // stride between split-K partial sums

  // Sum the partials in split order.  A chunk of up to four ranges is
  // loaded for all of the lane's experts before the first add, so those
  // loads are in flight together: one memory latency per chunk rather than
  // one per load.
  float z[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) z[v] = 0.f;
  for (int sp = 0; sp < a.ksplit; sp += 4) {
    float p[NV][4];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e = min(lane + 64 * v, a.E - 1);  // lanes past E load a valid entry, unused
#pragma unroll
      for (int u = 0; u < 4; ++u) p[v][u] = zrow[(size_t)min(sp + u, a.ksplit - 1) * zsplit + e];
    }
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (sp + u < a.ksplit) z[v] += p[v][u];
  }
  uint64_t key[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e = lane + 64 * v;
    if (e >= a.E) z[v] = -INFINITY;
    key[v] = (e < a.E) ? (((uint64_t)ordered_bits(z[v]) << 32) | (uint32_t)(~e)) : 0ull;
  }

  // softmax statistics over all E experts (max and sum of exp)
  float zmax = -INFINITY;
#pragma unroll
  for (int v = 0; v < NV; ++v) zmax = fmaxf(zmax, z[v]);
  zmax = wave_max(zmax);
  float esum = 0.f;
  if (a.score == 0) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
      if (lane + 64 * v < a.E) esum += expf(z[v] - zmax);
    esum = wave_sum(esum);
  }

  if (a.n_group > 0) {
    const int G = a.E / a.n_group;
    auto score = [&](int v) { return (a.score == 0) ? expf(z[v] - zmax) / esum : 1.f / (1.f + expf(-z[v])); };
    if ((G & (G - 1)) == 0 && G <= 64 && a.E % 64 == 0) {
      // Groups of a power-of-two size that tile the 64-expert columns: group
      // (lane + 64 v) / G is a segment of G lanes of column v.  Each lane
      // merges (largest, second largest) pairs with its partners at xor
      // distances 1 .. G/2, so every lane of a segment ends with its group's
      // two largest scores; the group scores are then read from one lane
      // of each segment and ranked in every lane.  No LDS, no barrier.
      float gs[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float b0 = score(v), b1 = -INFINITY;
        for (int off = 1; off < G; off <<= 1) {
          const float o0 = __shfl_xor(b0, off, 64), o1 = __shfl_xor(b1, off, 64);
          b1 = fmaxf(fminf(b0, o0), fmaxf(b1, o1));
          b0 = fmaxf(b0, o0);
        }
        gs[v] = b0 + b1;
      }
      const int per = 64 / G;  // groups per column
      int rank[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) rank[v] = 0;
#pragma unroll
      for (int vg = 0; vg < NV; ++vg)
        for (int q = 0; q < per; ++q) {
          const int g = vg * per + q;
          const float o = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gs[vg]), q * G));
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            const int gm = (lane + 64 * v) / G;
            rank[v] += (o > gs[v]) || (o == gs[v] && g < gm);
          }
        }
#pragma unroll
      for (int v = 0; v < NV; ++v)
        if (rank[v] >= a.topk_group) key[v] = 0ull;
    } else {
      // Any other grouping: scores through LDS, one lane per group.
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int e = lane + 64 * v;
        if (e < a.E) s_score[wave][e] = score(v);
      }
      __syncthreads();
      if (lane < a.n_group) {
        float b0 = -INFINITY, b1 = -INFINITY;  // two largest scores of the group
        for (int i = 0; i < G; ++i) {
          const float s = s_score[wave][lane * G + i];
          if (s > b0) { b1 = b0; b0 = s; } else if (s > b1) { b1 = s; }
        }
        s_gscore[wave][lane] = b0 + b1;
      }
      __syncthreads();
      if (lane < a.n_group) {
        const float mine = s_gscore[wave][lane];
        int rank = 0;
        for (int g = 0; g < a.n_group; ++g) {
          const float o = s_gscore[wave][g];
          rank += (o > mine) || (o == mine && g < lane);
        }
        s_keep[wave][lane] = rank < a.topk_group;
      }
      __syncthreads();
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int e = lane + 64 * v;
        if (e < a.E && !s_keep[wave][e / G]) key[v] = 0ull;
      }
    }
  }

  // top-k: k rounds of wave-wide maximum; the owner retires the winner.
  // With reroute candidates, k more rounds rank the next eligible experts
  // (a round whose maximum is 0 found none left).
  const int rounds = a.cand_idx ? 2 * a.k : a.k;
  uint64_t mine_key = 0ull;  // lane j keeps the j-th winner
  for (int j = 0; j < rounds; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int v = 0; v < NV; ++v) best = key[v] > best ? key[v] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int v = 0; v < NV; ++v)
      if (best != 0ull && key[v] == best) key[v] = 0ull;
    if (lane == j) mine_key = best;
  }

  const bool sel = lane < a.k;
  const bool cand = !sel && lane < rounds && mine_key != 0ull;
  const int e_sel = (int)(~(uint32_t)mine_key);
  const float z_sel = from_ordered_bits((uint32_t)(mine_key >> 32));
  // raw scores of the chosen (and candidate) experts; gates divide by the sum
  // over the chosen k (renorm), by the softmax sum, or by 1
  float r = 0.f;
  if (sel || cand) r = (a.score == 0) ? expf(z_sel - zmax) : 1.f / (1.f + expf(-z_sel));
  float denom = 1.f;
  if (a.renorm) denom = wave_sum(sel ? r : 0.f);
  else if (a.score == 0) denom = esum;
  const float g = r / denom;
  if (live && sel) {
    a.topk_idx[(size_t)t * a.k + lane] = e_sel;
    a.topk_w[(size_t)t * a.k + lane] = g;
  }
  if (live && a.cand_idx && !sel && lane < rounds) {
    a.cand_idx[(size_t)t * a.k + lane - a.k] = cand ? e_sel : -1;
    a.cand_w[(size_t)t * a.k + lane - a.k] = cand ? g : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Few experts (E <= 8, no group limit, bf16): the whole router in one kernel.
// A block takes TB = 64 / EM tokens; its four wavefronts split d into four
// ranges, and each lane runs over 16-byte chunks of its wavefront's range
// (lane-strided), loading each chunk for the E router rows and the TB tokens
// and accumulating the E x TB dot products with the packed bf16 dot
// instruction (fp32 accumulate).  The 4 x 64 partial sums of each product go
// through LDS; each wavefront adds a quarter of them and wavefront 0's lane
// l = tb * EM + e adds the four quarters, a fixed order for every product
// (identical router rows give identical logits), so token tb's logits
// sit in lanes [tb * EM, tb * EM + EM).  Scores, top-k and gates follow in
// those lane groups with shuffles that stay inside the group.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// A dword as two bf16.  Taken by value: a bit cast applied directly to a
// component of a vector (v.y) compiles to a cast of its first component.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// acc + sum of the 8 bf16 products of two 16-byte chunks (packed dot, fp32
// accumulate, pairs in element order).
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.w), acc, false);
  return acc;
}

template <int EM>
__global__ __launch_bounds__(256) void router_fused_kernel(RouterFusedArgs a) {
  constexpr int TB = 64 / EM;  // tokens per block
  __shared__ float s_part[4][64][65];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TB;
  const int nch = a.d / 8;  // 16-byte chunks per row
  const int c_lo = wave * nch / 4, c_hi = (wave + 1) * nch / 4;
  float acc[EM][TB];
#pragma unroll
  for (int e = 0; e < EM; ++e)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[e][j] = 0.f;
  const u32x4* wr = (const u32x4*)a.w_router;
  const u32x4* x = (const u32x4*)a.x;
  for (int c = c_lo + lane; c < c_hi; c += 64) {
    // every load unconditional (rows past E or T clamped, their products
    // unused), so a lane's 2 * TB loads are in flight together
    u32x4 xv[TB], wv[EM];
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int t = min(t0 + j, a.T - 1);
      xv[j] = x[(size_t)t * nch + c];
    }
#pragma unroll
    for (int e = 0; e < EM; ++e) wv[e] = wr[(size_t)min(e, a.E - 1) * nch + c];
#pragma unroll
    for (int e = 0; e < EM; ++e)
#pragma unroll
      for (int j = 0; j < TB; ++j) acc[e][j] = dot8(wv[e], xv[j], acc[e][j]);
  }
#pragma unroll
  for (int e = 0; e < EM; ++e)
#pragma unroll
    for (int j = 0; j < TB; ++j) s_part[wave][lane][j * EM + e] = acc[e][j];
  __syncthreads();
  // entry i = threadIdx.x % 64 summed by all four waves: wave q adds lanes
  // [16q, 16q + 16) of every wave's range, then wave 0 adds the four sums
  // (a fixed order for every entry)
  {
    const int q = wave, i = lane;
    float p = 0.f;
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int l = 0; l < 16; ++l) p += s_part[w][16 * q + l][i];
    __syncthreads();  // every read of s_part is done before the slots are reused
    s_part[0][q][i] = p;
  }
  __syncthreads();
  if (wave != 0) return;
  float z = 0.f;  // entry `lane` summed over the four quarters
  for (int q = 0; q < 4; ++q) z += s_part[0][q][lane];
  const int e = lane % EM, tb = lane / EM, t = t0 + tb;
  const bool real = e < a.E;
  if (real && a.bias) z += a.bias[e];
  // group reductions over the EM lanes of a token (xor offsets < EM stay inside)
  auto gmax = [&](float v) {
#pragma unroll
    for (int off = EM / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
  };
  auto gsum = [&](float v) {
#pragma unroll
    for (int off = EM / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
  };
  auto gmax_u64 = [&](uint64_t v) {
#pragma unroll
    for (int off = EM / 2; off >= 1; off >>= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off, 64);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off, 64);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      v = o > v ? o : v;
    }
    return v;
  };
  const float zl = real ? z : -INFINITY;
  const float zmax = gmax(zl);
  const float esum = (a.score == 0) ? gsum(real ? expf(zl - zmax) : 0.f) : 0.f;
  uint64_t key = real ? (((uint64_t)ordered_bits(z) << 32) | (uint32_t)(~e)) : 0ull;
  // rank of this lane's expert among the token's (k rounds; 2k with candidates)
  const int rounds = a.cand_idx ? 2 * a.k : a.k;
  int rank = -1;
  for (int j = 0; j < rounds; ++j) {
    const uint64_t best = gmax_u64(key);
    if (best != 0ull && key == best) {
      rank = j;
      key = 0ull;
    }
  }
  const bool sel = rank >= 0 && rank < a.k;
  const bool cand = rank >= a.k;
  float r = 0.f;
  if (sel || cand) r = (a.score == 0) ? expf(z - zmax) : 1.f / (1.f + expf(-z));
  float denom = 1.f;
  if (a.renorm) denom = gsum(sel ? r : 0.f);
  else if (a.score == 0) denom = esum;
  const float g = r / denom;
  if (t < a.T && sel) {
    a.topk_idx[(size_t)t * a.k + rank] = e;
    a.topk_w[(size_t)t * a.k + rank] = g;
  }
  if (t < a.T && a.cand_idx) {
    if (cand) {
      a.cand_idx[(size_t)t * a.k + rank - a.k] = e;
      a.cand_w[(size_t)t * a.k + rank - a.k] = g;
    }
    // ranks past the experts there are: no candidate
    if (e == 0)
      for (int m = max(a.E - a.k, 0); m < a.k; ++m) {
        a.cand_idx[(size_t)t * a.k + m] = -1;
        a.cand_w[(size_t)t * a.k + m] = 0.f;
      }
  }
}

}  // namespace

// Every block re-reads all of Wr for its 64 / E' tokens, so Wr traffic is
// (E / (64 / E')) times that of x: at most x's for E <= 8.  Wider routers
// stay on the split-K GEMM.
bool router_fused_ok(int T, int d, int E, int k, int n_group, int act) {
  return act == GD_BF16 && E <= 8 && n_group == 0 && k <= E && T > 0 && d % 8 == 0;
}

hipError_t launch_router_fused(const RouterFusedArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int em = a.E <= 8 ? 8 : a.E <= 16 ? 16 : 32;
  const int per_block = 64 / em;  // tokens per block
  const dim3 grid((a.T + per_block - 1) / per_block);
  if (em == 8) hipLaunchKernelGGL(router_fused_kernel<8>, grid, dim3(256), 0, s, a);
  else if (em == 16) hipLaunchKernelGGL(router_fused_kernel<16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(router_fused_kernel<32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_route_select(const RouteSelectArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int blocks = (a.T + kWaves - 1) / kWaves;
  switch ((a.E + 63) / 64) {
    case 1: hipLaunchKernelGGL(route_select_kernel<1>, dim3(blocks), dim3(kWaves * 64), 0, s, a); break;
    case 2: hipLaunchKernelGGL(route_select_kernel<2>, dim3(blocks), dim3(kWaves * 64), 0, s, a); break;
    case 3: hipLaunchKernelGGL(route_select_kernel<3>, dim3(blocks), dim3(kWaves * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL(route_select_kernel<4>, dim3(blocks), dim3(kWaves * 64), 0, s, a); break;
    case 5: hipLaunchKernelGGL(route_select_kernel<5>, dim3(blocks), dim3(kWaves * 64), 0, s, a); break;
    case 6: hipLaunchKernelGGL(route_select_kernel<6>, dim3(blocks), dim3(kWaves * 64), 0, s, a); break;
    case 7: hipLaunchKernelGGL(route_select_kernel<7>, dim3(blocks), dim3(kWaves * 64), 0, s, a); break;
    case 8: hipLaunchKernelGGL(route_select_kernel<8>, dim3(blocks), dim3(kWaves * 64), 0, s, a); break;
    default: return hipErrorInvalidValue;  // E > kMaxE: the caller checks
  }
  return hipGetLastError();
}

}  // namespace moe
