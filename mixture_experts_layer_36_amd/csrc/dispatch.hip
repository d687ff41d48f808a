// Dispatch: per-expert histogram, exclusive scan, stable permutation into
// expert-contiguous rows, and the row gather that fills the dispatch buffer.
//
// The expert-contiguous buffer is the layout the dispatch exchange ships to
// the expert owners ("Expert-Parallel MoE Inference: Serving Sparse Models at
// Scale", section "The all-to-all dispatch and combine, step by step",
// Figure 3); counts[e] are the per-expert token counts that page's checklist
// asks to export (section "Trade-offs, Gotchas, and What Goes Wrong").
//
// Three index kernels, all deterministic (no result depends on atomic order)
// (up to 4096 assignments, one block does all three: dispatch_small_kernel):
//   1. histogram: one wavefront per chunk of a.chunk assignments,
//      LDS-privatised bins -> chunk_cnt[chunk][e];
//   2. scan (one block): per-expert running sums over chunks give each
//      chunk's first row per expert; an exclusive scan over experts gives
//      offsets;
//   3. scatter: one wavefront per chunk walks its assignments in order, 64 at
//      a time; a lane's rank among earlier lanes with the same expert comes
//      from ballot equality masks, so rows within an expert follow the
//      assignment order a = t*k + j (increasing token).
//
// With a capacity and overflow rerouted ("Expert-Parallel MoE Inference",
// section "Capacity factor and token dropping": overflow goes to the token's
// next-best expert) the dispatch runs two passes:
//   1. histogram and scan as above; the scatter only ranks each assignment
//      within its own expert (rank < capacity: it keeps a slot there);
//   2. per token, its m-th overflowed assignment (increasing j) is offered
//      the token's candidate m; a histogram and a scan of the offers per
//      expert against the slots pass 1 left, then one scatter lays out each
//      expert's pass-1 rows followed by its accepted offers, both in
//      increasing a.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kMaxE = 512;
constexpr int kIdBits = 10;  // ids 0..512 (512 marks an idle lane)

// keys[i] in [0, E), or negative (not counted); per-chunk counts to out.
__global__ __launch_bounds__(64) void histogram_kernel(DispatchArgs a, const int32_t* keys, int32_t* out) {
  __shared__ int bins[kMaxE];
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E; e += 64) bins[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * a.chunk;
  const int end = min(base + a.chunk, a.n_assign);
  for (int i = base + lane; i < end; i += 64) {
    const int e = keys[i];
    if (e >= 0) atomicAdd(&bins[e], 1);
  }
  __syncthreads();
  for (int e = lane; e < a.E; e += 64) out[(size_t)blockIdx.x * a.E + e] = bins[e];
}

__global__ __launch_bounds__(kMaxE) void scan_kernel(DispatchArgs a, int n_chunks) {
  __shared__ int tot[kMaxE];
  const int e = threadIdx.x;
  int run = 0;
  if (e < a.E) {
    // rows of e before chunk c (relative to offsets[e]); the chunk counts are
    // read 16 at a time so their loads are in flight together
    constexpr int kBatch = 16;
    int c0 = 0;
    for (; c0 + kBatch <= n_chunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = a.chunk_cnt[(size_t)(c0 + u) * a.E + e];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        a.chunk_cnt[(size_t)(c0 + u) * a.E + e] = run;
        run += v[u];
      }
    }
    for (int c = c0; c < n_chunks; ++c) {
      int* p = a.chunk_cnt + (size_t)c * a.E + e;
      const int v = *p;
      *p = run;
      run += v;
    }
    a.counts[e] = run;  // the demand; the rows kept are min(run, cap)
  }
  const int kept = (e < a.E) ? min(run, a.cap) : 0;
  tot[e] = kept;
  __syncthreads();
  // inclusive Hillis-Steele scan over kMaxE entries
  for (int off = 1; off < kMaxE; off <<= 1) {
    const int v = (e >= off) ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  const int excl = tot[e] - kept;
  if (e < a.E) a.offsets[e] = excl;  // the scatter adds it to the relative chunk bases
  if (e == a.E - 1) a.offsets[a.E] = tot[e];
}

// rank_out == NULL: rows and inv_pos as described above.  Otherwise only the
// rank of each assignment within its expert goes to rank_out (pass 1 of the
// rerouting dispatch).
__global__ __launch_bounds__(64) void scatter_kernel(DispatchArgs a, int32_t* rank_out) {
  __shared__ int next_row[kMaxE];  // rank within the expert of the chunk's next assignment
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E; e += 64) next_row[e] = a.chunk_cnt[(size_t)blockIdx.x * a.E + e];
  __syncthreads();
  const int base = blockIdx.x * a.chunk;
  const int end = min(base + a.chunk, a.n_assign);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s = base; s < end; s += 64) {
    const int i = s + lane;
    const bool valid = i < end;
    const int e = valid ? a.topk_idx[i] : kMaxE;
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < kIdBits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & below);
    const int rel = valid ? next_row[e] + rank : 0;  // earlier assignments to e
    __syncthreads();  // every lane has read next_row before any update
    const bool last = (same >> lane) == 1ull;  // highest lane of its group
    if (valid && last) next_row[e] = rel + 1;
    __syncthreads();
    if (valid && rank_out) {
      rank_out[i] = rel;
    } else if (valid) {
      if (rel < a.cap) {  // a free slot of its expert
        const int row = a.offsets[e] + rel;
        a.inv_pos[i] = row;
        a.perm_token[row] = i / a.k;
      } else {
        a.inv_pos[i] = -1;  // the expert is full: dropped
      }
    }
  }
}

// Small problems (at most kSmallDispatch assignments): histogram, scan and
// scatter in one block of 8 wavefronts, the arithmetic of the three kernels
// above with one chunk per wavefront.  The expert ids are staged in LDS
// once; each wave bins its chunk (LDS atomics: integer, order-free); thread e
// turns the 8 chunk counts of expert e into chunk bases and the scan over
// experts gives the offsets; then every wave walks its own chunk in order, 64
// at a time, ranking each lane among earlier lanes with the same expert by
// ballots.  One launch instead of three, which is most of the cost at decode
// sizes.
constexpr int kSmallDispatch = 4096, kSmallWaves = kMaxE / 64;
__global__ __launch_bounds__(kMaxE) void dispatch_small_kernel(DispatchArgs a) {
  __shared__ int keys[kSmallDispatch];
  __shared__ int cnt[kSmallWaves][kMaxE];  // per chunk: counts, then its next row per expert
  __shared__ int tot[kMaxE];
  __shared__ int base[kMaxE];              // first row of each expert
  const int e = threadIdx.x, wave = e >> 6, lane = e & 63;
  for (int i = e; i < a.n_assign; i += kMaxE) keys[i] = a.topk_idx[i];
  for (int w = 0; w < kSmallWaves; ++w) cnt[w][e] = 0;
  __syncthreads();
  // chunk w: assignments [w * C, min((w + 1) * C, n)), C a multiple of 64
  const int C = ((a.n_assign + kSmallWaves * 64 - 1) / (kSmallWaves * 64)) * 64;
  const int lo = min(wave * C, a.n_assign), hi = min(lo + C, a.n_assign);
  for (int i = lo + lane; i < hi; i += 64) {
    const int x = keys[i];
    if (x >= 0) atomicAdd(&cnt[wave][x], 1);
  }
  __syncthreads();
  int run = 0;
  if (e < a.E) {
    for (int w = 0; w < kSmallWaves; ++w) {
      const int v = cnt[w][e];
      cnt[w][e] = run;  // rows of e before chunk w (relative)
      run += v;
    }
    a.counts[e] = run;  // the demand; the rows kept are min(run, cap)
  }
  const int kept = (e < a.E) ? min(run, a.cap) : 0;
  tot[e] = kept;
  __syncthreads();
  for (int off = 1; off < kMaxE; off <<= 1) {
    const int v = (e >= off) ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  base[e] = tot[e] - kept;
  if (e < a.E) a.offsets[e] = tot[e] - kept;
  if (e == a.E - 1) a.offsets[a.E] = tot[e];
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* next_row = cnt[wave];
  for (int s0 = lo; s0 < hi; s0 += 64) {
    const int i = s0 + lane;
    const bool valid = i < hi;
    const int x = valid ? keys[i] : kMaxE;
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < kIdBits; ++b) {
      const bool bit = (x >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & below);
    const int rel = valid ? next_row[x] + rank : 0;  // earlier assignments to x
    __builtin_amdgcn_wave_barrier();  // every lane has read next_row before any update
    const bool last = (same >> lane) == 1ull;  // highest lane of its group
    if (valid && last) next_row[x] = rel + 1;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      if (rel < a.cap) {  // a free slot of its expert
        const int row = base[x] + rel;
        a.inv_pos[i] = row;
        a.perm_token[row] = i / a.k;
      } else {
        a.inv_pos[i] = -1;  // the expert is full: dropped
      }
    }
  }
}

// Pass 2 offers, one thread per token: the m-th assignment of the token that
// found its own expert full (increasing j) is offered candidate m; the gate of
// every assignment is that of the copy that would serve it.
__global__ __launch_bounds__(256) void reroute_offer_kernel(DispatchArgs a, RerouteArgs r, int T) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int m = 0;
  for (int j = 0; j < a.k; ++j) {
    const int i = t * a.k + j;
    if (r.rel[i] < a.cap) {
      r.target[i] = -1;
      r.gate[i] = r.topk_w[i];
    } else {
      r.target[i] = r.cand_idx[t * a.k + m];
      r.gate[i] = r.cand_w[t * a.k + m];
      ++m;
    }
  }
}

// Pass 2 scan: per expert, the offers before each chunk (relative), how many
// fit in the slots pass 1 left, and the offsets of pass-1 + pass-2 rows.
__global__ __launch_bounds__(kMaxE) void reroute_scan_kernel(DispatchArgs a, RerouteArgs r, int n_chunks) {
  __shared__ int tot[kMaxE];
  const int e = threadIdx.x;
  int run = 0, kept = 0;
  if (e < a.E) {
    for (int c = 0; c < n_chunks; ++c) {
      int* p = r.chunk_cnt2 + (size_t)c * a.E + e;
      const int v = *p;
      *p = run;
      run += v;
    }
    const int kept1 = min(a.counts[e], a.cap);
    kept = kept1 + min(run, a.cap - kept1);
  }
  tot[e] = kept;
  __syncthreads();
  for (int off = 1; off < kMaxE; off <<= 1) {
    const int v = (e >= off) ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < a.E) a.offsets[e] = tot[e] - kept;
  if (e == a.E - 1) a.offsets[a.E] = tot[e];
}

// Pass 2 scatter: an assignment ranked below the capacity takes row
// offsets[e] + rank; an offer to c takes row offsets[c] + kept1[c] + its rank
// among the offers to c, if that is below the slots pass 1 left; anything
// else is dropped.  Offer ranks follow a, as in scatter_kernel.
__global__ __launch_bounds__(64) void reroute_scatter_kernel(DispatchArgs a, RerouteArgs r) {
  __shared__ int next_row[kMaxE];
  const int lane = threadIdx.x;
  for (int e = lane; e < a.E; e += 64) next_row[e] = r.chunk_cnt2[(size_t)blockIdx.x * a.E + e];
  __syncthreads();
  const int base = blockIdx.x * a.chunk;
  const int end = min(base + a.chunk, a.n_assign);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s = base; s < end; s += 64) {
    const int i = s + lane;
    const bool valid = i < end;
    const int c = valid ? r.target[i] : -1;
    const int key = c >= 0 ? c : kMaxE;  // kMaxE: not an offer
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < kIdBits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & below);
    const int rel2 = (c >= 0) ? next_row[c] + rank : 0;
    __syncthreads();
    const bool last = (same >> lane) == 1ull;
    if (c >= 0 && last) next_row[c] = rel2 + 1;
    __syncthreads();
    if (!valid) continue;
    const int rel = r.rel[i];
    if (rel < a.cap) {
      const int row = a.offsets[a.topk_idx[i]] + rel;
      a.inv_pos[i] = row;
      a.perm_token[row] = i / a.k;
    } else if (c >= 0) {
      const int kept1 = min(a.counts[c], a.cap);
      if (rel2 < a.cap - kept1) {
        const int row = a.offsets[c] + kept1 + rel2;
        a.inv_pos[i] = row;
        a.perm_token[row] = i / a.k;
      } else {
        a.inv_pos[i] = -1;
      }
    } else {
      a.inv_pos[i] = -1;
    }
  }
}

// x_perm[p][:] = x[perm_token[p]][:], 16-byte vectors; one block per 8 rows.
// rows_dev (device, nullable): the number of rows actually laid out
// (offsets[E]), at most `rows`; rows past it are left untouched.
__global__ __launch_bounds__(256) void gather_kernel(const u32x4* __restrict__ x,
                                                     const int32_t* __restrict__ perm,
                                                     int rows, const int32_t* __restrict__ rows_dev,
                                                     int vec_per_row, u32x4* __restrict__ out) {
  const int r0 = blockIdx.x * 8;
  const int n = rows_dev ? min(*rows_dev, rows) : rows;
  for (int r = r0; r < min(r0 + 8, n); ++r) {
    const size_t src = (size_t)perm[r] * vec_per_row;
    const size_t dst = (size_t)r * vec_per_row;
    for (int v = threadIdx.x; v < vec_per_row; v += 256) out[dst + v] = x[src + v];
  }
}

// The same rows into K/pw planes of [rows][pw] bf16 (perm NULL: x's rows in
// order): thread g moves the 16 bytes at g, so a wave stores one contiguous
// kilobyte (16 rows x 64 bytes, or 8 rows x 128, of one plane) and loads
// 16 (8) row runs.
__global__ __launch_bounds__(256) void gather_blocked_kernel(const u32x4* __restrict__ x,
                                                             const int32_t* __restrict__ perm, int rows,
                                                             const int32_t* __restrict__ rows_dev, int d,
                                                             int pw, u32x4* __restrict__ out) {
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = pw / 8;  // 16-byte chunks per row and plane
  const size_t per_plane = (size_t)rows * cpr;
  if (g >= per_plane * (d / pw)) return;
  // The token-order copy (no row map) walks x row by row, consecutive threads
  // on consecutive 16-byte chunks of a row (Qwen-shaped copy: dispatch stage
  // 61 -> 54 us); the gather of x_perm walks the planes, which suited it
  // better (the row walk cost the Mixtral-shaped gather 8%).
  int p, r, q;
  if (perm == nullptr) {
    const int cpx = d / 8, cx = (int)(g % cpx);
    r = (int)(g / cpx);
    p = cx / cpr;
    q = cx % cpr;
  } else {
    const int rem = (int)(g % per_plane);
    p = (int)(g / per_plane);
    r = rem / cpr;
    q = rem % cpr;
  }
  const int n = rows_dev ? min(*rows_dev, rows) : rows;
  if (r >= n) return;
  out[(size_t)p * per_plane + (size_t)r * cpr + q] = x[((size_t)(perm ? perm[r] : r) * d + p * pw + q * 8) / 8];
}

__global__ __launch_bounds__(256) void segment_rows_kernel(const int32_t* offsets, int E, int32_t* rows) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < E) rows[e] = offsets[e + 1] - offsets[e];
}

__global__ void zero_counts_kernel(DispatchArgs a) {
  const int e = threadIdx.x;
  if (e < a.E) a.counts[e] = 0;
  if (a.offsets != nullptr && e <= a.E) a.offsets[e] = 0;
}

}  // namespace

hipError_t launch_dispatch_index(const DispatchArgs& a_in, hipStream_t s) {
  DispatchArgs a = a_in;
  a.chunk = dispatch_chunk(a.n_assign);
  if (a.n_assign == 0) {  // a fill kernel, not a memset node (graph-safe)
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(kMaxE + 64), 0, s, a);
    return hipGetLastError();
  }
  if (a.n_assign <= kSmallDispatch) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kMaxE), 0, s, a);
    return hipGetLastError();
  }
  const int n_chunks = (a.n_assign + a.chunk - 1) / a.chunk;
  hipLaunchKernelGGL(histogram_kernel, dim3(n_chunks), dim3(64), 0, s, a, a.topk_idx, a.chunk_cnt);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kMaxE), 0, s, a, n_chunks);
  hipLaunchKernelGGL(scatter_kernel, dim3(n_chunks), dim3(64), 0, s, a, (int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_dispatch_reroute(const DispatchArgs& a_in, const RerouteArgs& r, hipStream_t s) {
  if (a_in.n_assign == 0) return launch_dispatch_index(a_in, s);
  DispatchArgs a = a_in;
  a.chunk = dispatch_chunk(a.n_assign);
  const int n_chunks = (a.n_assign + a.chunk - 1) / a.chunk;
  const int T = a.n_assign / a.k;
  hipLaunchKernelGGL(histogram_kernel, dim3(n_chunks), dim3(64), 0, s, a, a.topk_idx, a.chunk_cnt);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kMaxE), 0, s, a, n_chunks);
  hipLaunchKernelGGL(scatter_kernel, dim3(n_chunks), dim3(64), 0, s, a, r.rel);
  hipLaunchKernelGGL(reroute_offer_kernel, dim3((T + 255) / 256), dim3(256), 0, s, a, r, T);
  hipLaunchKernelGGL(histogram_kernel, dim3(n_chunks), dim3(64), 0, s, a, (const int32_t*)r.target,
                     r.chunk_cnt2);
  hipLaunchKernelGGL(reroute_scan_kernel, dim3(1), dim3(kMaxE), 0, s, a, r, n_chunks);
  hipLaunchKernelGGL(reroute_scatter_kernel, dim3(n_chunks), dim3(64), 0, s, a, r);
  return hipGetLastError();
}

hipError_t launch_segment_rows(const int32_t* offsets, int E, int32_t* rows, hipStream_t s) {
  hipLaunchKernelGGL(segment_rows_kernel, dim3((E + 255) / 256), dim3(256), 0, s, offsets, E, rows);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* perm_token, int rows, const int32_t* rows_dev,
                              int row_bytes, void* x_perm, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3((rows + 7) / 8), dim3(256), 0, s,
                     (const u32x4*)x, perm_token, rows, rows_dev, row_bytes / 16, (u32x4*)x_perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows_blocked(const void* x, const int32_t* perm_token, int rows, const int32_t* rows_dev,
                                      int d, int pw, void* x_perm, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if ((pw != 32 && pw != 64) || d % pw != 0) return hipErrorInvalidValue;
  const size_t threads = (size_t)rows * (d / 8);
  hipLaunchKernelGGL(gather_blocked_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     (const u32x4*)x, perm_token, rows, rows_dev, d, pw, (u32x4*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
