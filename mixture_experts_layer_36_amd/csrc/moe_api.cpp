// C ABI of the MoE layer forward: host-side validation, workspace carving and
// launch order.  Every entry point validates all arguments before it enqueues
// anything, never allocates, never synchronises, and reports failures as
// moe_status codes.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <mutex>

#include "moe_internal.hpp"

using namespace moe;

// Scratch of moe_dispatch_noalloc: the per-chunk expert counts of the
// dispatch index kernels, in a static device array (one copy per GPU, held
// until the process ends) instead of a caller workspace.  Host code never
// uses the symbol itself as an address: each device's copy is looked up once
// with hipGetSymbolAddress (scratch_on_current_device) and that pointer is
// what the kernels get.
static __device__ __align__(256) int32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxE = 512;
constexpr int kMaxK = 16;
constexpr int kMaxGroups = 64;
constexpr int64_t kMaxAssign = int64_t(1) << 28;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

size_t act_bytes(const moe_desc* d) { return d->act == MOE_F32 ? 4 : 2; }

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a required pointer: non-null and 16-byte aligned
bool need(const void* p) { return p != nullptr && aligned(p); }
// a nullable pointer: null, or 16-byte aligned
bool maybe(const void* p) { return p == nullptr || aligned(p); }

moe_status check_desc(const moe_desc* d) {
  if (d == nullptr) return MOE_ERR_INVALID;
  if (d->T < 0 || d->d <= 0 || d->f <= 0 || d->E <= 0 || d->k <= 0 || d->f_shared < 0)
    return MOE_ERR_INVALID;
  if (d->k > d->E) return MOE_ERR_INVALID;
  if (d->score != MOE_SCORE_SOFTMAX && d->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID;
  if (d->renorm != 0 && d->renorm != 1) return MOE_ERR_INVALID;
  if (d->act != MOE_F32 && d->act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->wdtype != MOE_F32 && d->wdtype != MOE_BF16 && d->wdtype != MOE_FP8_E4M3)
    return MOE_ERR_INVALID;
  if (d->act == MOE_F32 && d->wdtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (d->act == MOE_BF16 && d->wdtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (d->n_group < 0 || d->topk_group < 0) return MOE_ERR_INVALID;
  if (d->n_group > 0) {
    if (d->E % d->n_group != 0 || d->E / d->n_group < 2) return MOE_ERR_INVALID;
    if (d->topk_group < 1 || d->topk_group > d->n_group) return MOE_ERR_INVALID;
    if (int64_t(d->topk_group) * (d->E / d->n_group) < d->k) return MOE_ERR_INVALID;
    if (d->n_group > kMaxGroups) return MOE_ERR_UNSUPPORTED;
  }
  if (d->E > kMaxE || d->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (d->d % 128 != 0 || d->f % 128 != 0 || d->f_shared % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (int64_t(d->T) * d->k >= kMaxAssign) return MOE_ERR_UNSUPPORTED;
  if (d->capacity < 0) return MOE_ERR_INVALID;
  if (d->overflow != MOE_OVERFLOW_DROP && d->overflow != MOE_OVERFLOW_REROUTE) return MOE_ERR_INVALID;
  if (d->dispatch_fp8 != 0 && d->dispatch_fp8 != 1) return MOE_ERR_INVALID;
  if (d->dispatch_fp8 && d->act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->w_layout != MOE_W_ROWMAJOR && d->w_layout != MOE_W_KBLOCKED) return MOE_ERR_INVALID;
  if (d->w_layout == MOE_W_KBLOCKED) {
    // bf16 / fp8 expert kernels only; each matrix within the kernels' 32-bit
    // buffer offsets
    if (d->wdtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
    const int64_t wb = d->wdtype == MOE_BF16 ? 2 : 1;
    if (int64_t(d->d) * d->f * wb >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int64_t n_assign(const moe_desc* d) { return int64_t(d->T) * d->k; }

// Capacity overflow rerouted to the next-best expert (moe_layer_forward).
bool reroute(const moe_desc* d) { return d->capacity > 0 && d->overflow == MOE_OVERFLOW_REROUTE; }

int gemm_dtype(int moe_dt) {
  return moe_dt == MOE_F32 ? GD_F32 : moe_dt == MOE_BF16 ? GD_BF16 : GD_FP8;
}

// The fp8 dispatch payload of R rows: codes, then scales (moe.h).
size_t payload_sstride(const moe_desc* d) { return MOE_FP8_SCALE_STRIDE(d->d); }
size_t payload_bytes(const moe_desc* d, size_t R) { return MOE_FP8_PAYLOAD_BYTES(R, d->d); }
uint8_t* payload_scales(void* p, const moe_desc* d, size_t R) {
  return static_cast<uint8_t*>(p) + MOE_FP8_SCALES_OFFSET(R, d->d);
}

// The gate-up GEMM runs fp8 x fp8 on the payload itself (E4M3 weights on a
// prefill-shaped problem); otherwise it reads the payload's values as bf16.
bool fp8_act(const moe_desc* d) {
  if (!d->dispatch_fp8 || d->wdtype != MOE_FP8_E4M3) return false;
  GemmArgs g{};
  g.act = GD_FP8;
  g.wdt = GD_FP8;
  g.epi = EPI_SWIGLU;
  g.rows = int(int64_t(d->T) * d->k);
  g.E = d->E;
  g.K = d->d;
  g.a_sstride = int(payload_sstride(d));
  return gemm_fp8_act_ok(g);
}

// m-tile height of the routed grouped GEMMs (must match the launch)
int block_m(const moe_desc* d) {
  GemmArgs g{};
  g.act = gemm_dtype(d->act);
  g.wdt = gemm_dtype(d->wdtype);
  g.rows = int(int64_t(d->T) * d->k);
  g.E = d->E;
  g.epi = EPI_SWIGLU;
  return gemm_block_m(g);
}

// ---------------------------------------------------------------- workspace
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align_up(bytes);
    return p;
  }
};

struct RouteWs {
  float* z;    // [ksplit][T][E] partial logits
  int ksplit;
  int32_t* cand_idx;  // reroute candidates [T][k] (NULL: not rerouting)
  float* cand_w;
};

// The router GEMM on the prefill kernel: tiles of 256 rows (or 128), 256 or
// 128 experts wide, K split until one wave of the GPU is filled, each range
// at least 8 stages of 32 and the partial sums at most twice the input.
// 128-row tiles where 256-row ones would need ranges shorter than 32 stages:
// the tile's fixed cost then outweighs its loop (Qwen-shaped route, 16-stage
// ranges: 52 -> 43 us on 128-row tiles; DeepSeek-V3-shaped, 56-stage ranges:
// 141 -> 152 us on them).
struct RouterPlan {
  int rows, ksplit;
};
RouterPlan big_router_plan(const moe_desc* d) {
  const int64_t in_bytes = (int64_t(d->T) + d->E) * d->d * 2;
  const int64_t part_bytes = int64_t(d->T) * d->E * 4;
  const int bn = d->E % 256 == 0 ? 256 : 128;
  RouterPlan p{256, 1};
  for (int rows : {256, 128}) {
    const int64_t tiles = int64_t((d->T + rows - 1) / rows) * ((d->E + bn - 1) / bn);
    int64_t want = (256 + tiles - 1) / tiles;
    want = std::min<int64_t>(want, std::max<int64_t>(1, 2 * in_bytes / std::max<int64_t>(part_bytes, 1)));
    want = std::min<int64_t>(want, std::max<int64_t>(1, d->d / 256));
    p = RouterPlan{rows, int(std::max<int64_t>(1, std::min<int64_t>(want, 16)))};
    if ((d->d / 32) / p.ksplit >= 32) break;
  }
  return p;
}

// Split-K factor of the router GEMM: enough blocks to fill the GPU when T*E
// is small (decode, few experts), bounded so the fp32 partial sums stay small
// next to the inputs.  K / ksplit stays a multiple of the 64-wide k step.
int route_splits(const moe_desc* d) {
  if (d->act == MOE_F32) return 1;
  GemmArgs g{};  // the launch the router GEMM will use
  g.act = gemm_dtype(d->act);
  g.wdt = gemm_dtype(d->act);
  g.rows = d->T;
  g.N = d->E;
  g.epi = EPI_BIAS_F32;
  const int bm = gemm_block_m(g);
  const int64_t in_bytes = (int64_t(d->T) + d->E) * d->d * 2;
  const int64_t part_bytes = int64_t(d->T) * d->E * 4;
  if (bm == 256) return big_router_plan(d).ksplit;
  const int64_t tiles = int64_t((d->T + 127) / 128) * ((d->E + 127) / 128);
  const int64_t kmax = d->d / 64;
  int64_t want = (1024 + tiles - 1) / tiles;
  want = std::min<int64_t>(want, std::max<int64_t>(1, 2 * in_bytes / std::max<int64_t>(part_bytes, 1)));
  // at most 16 ranges: more only multiplies the partial sums the selection
  // reads (DeepSeek-V3-shaped decode: 56 ranges 34.6 us, 16 ranges 26.6 us)
  want = std::min<int64_t>(want, 16);
  int s = 1;
  for (int64_t c = 1; c <= std::min(want, kmax); ++c)
    if (kmax % c == 0) s = int(c);
  return s;
}
struct DispatchWs {
  int32_t* chunk_cnt;
  RerouteArgs rr;     // rerouting workspace (pointers NULL when not rerouting)
};
struct FfnWs {
  int32_t* table;
  int n_slots;
  float* partial;     // K-split partial sums of the prefill kernel (NULL: not used)
  int partial_slots;
  int32_t* sched;     // block records of the prefill kernel (NULL: not used)
  int sched_cap;
};
struct LayerWs {
  RouteWs route;
  DispatchWs disp;
  FfnWs ffn;
  int32_t* perm_token;
  int32_t* inv_pos;
  int32_t* offsets;
  void* x_perm;
  void* xq;       // dispatch_fp8 with the fused gather: x's payload (or its bf16 values) in token order
  void* xb;       // x in K-blocked planes, token order (x_blocked)
  void* h;
  void* y_perm;
  void* sh;
  void* sy;
};

RouteWs carve_route(Carve& c, const moe_desc* d, bool with_candidates) {
  const int ks = route_splits(d);
  RouteWs w{c.take<float>(sizeof(float) * size_t(ks) * d->T * d->E), ks, nullptr, nullptr};
  if (with_candidates) {
    w.cand_idx = c.take<int32_t>(sizeof(int32_t) * size_t(n_assign(d)));
    w.cand_w = c.take<float>(sizeof(float) * size_t(n_assign(d)));
  }
  return w;
}
DispatchWs carve_dispatch(Carve& c, const moe_desc* d, bool rerouting) {
  const int64_t chunks = (n_assign(d) + kMinDispatchChunk - 1) / kMinDispatchChunk;
  DispatchWs w{};
  w.chunk_cnt = c.take<int32_t>(sizeof(int32_t) * size_t(chunks) * d->E);
  if (rerouting) {
    const size_t A = size_t(n_assign(d));
    w.rr.chunk_cnt2 = c.take<int32_t>(sizeof(int32_t) * size_t(chunks) * d->E);
    w.rr.rel = c.take<int32_t>(sizeof(int32_t) * A);
    w.rr.target = c.take<int32_t>(sizeof(int32_t) * A);
    w.rr.gate = c.take<float>(sizeof(float) * A);
  }
  return w;
}
// The shared expert joins the routed grouped GEMMs as one more segment when
// its weights have the routed weights' dtype.
bool fuse_shared(const moe_desc* d) { return d->f_shared > 0 && d->wdtype == d->act; }

FfnWs carve_ffn(Carve& c, const moe_desc* d, bool with_shared) {
  FfnWs w;
  w.n_slots = gemm_max_slots(int(n_assign(d)), d->E, block_m(d), with_shared ? d->T : 0);
  w.table = c.take<int32_t>(sizeof(int32_t) * size_t(w.n_slots + 1));
  w.partial = nullptr;
  w.partial_slots = 0;
  w.sched = nullptr;
  w.sched_cap = 0;
  if (block_m(d) == 256) {  // the prefill kernel splits its last wave of tiles
    w.partial = c.take<float>(kPartialSlotBytes * kPartialSlots);
    w.partial_slots = kPartialSlots;
    // one record per block of either routed GEMM: n-tiles of at least 128
    // output columns, plus a wave of K-pieces (at most one per compute unit;
    // 2048 covers any CU count the split plan can use)
    const int cols = std::max(std::max(d->f, d->f_shared), d->d);
    const int64_t cap = int64_t(w.n_slots) * ((cols + 127) / 128) + 2048;
    if (cap < (int64_t(1) << 30)) {
      w.sched = c.take<int32_t>(sizeof(int32_t) * kSchedInts * size_t(cap));
      w.sched_cap = int(cap);
    }
  }
  return w;
}

// The layer reads GEMM1's activation rows straight from x through perm_token
// (x_perm is never written) when every row offset of x fits the kernels'
// 32-bit buffer offsets.
// x_perm gathered into K-blocked planes instead of the fused gather: the
// gate-up GEMM's 256-row tiles then read whole 32-column slices of A as
// contiguous runs.  That saves ~4.5% of the GEMM (measured at d = 4096,
// f = 14336) and costs the gather's 2 * T*k * d * 2 bytes; the saving grows
// with d * f and the cost with d, so it pays from f ~ 4096 up.
bool gather_blocked(const moe_desc* d) {
  return d->act == MOE_BF16 && !d->dispatch_fp8 && d->f >= 4096 && block_m(d) == 256 &&
         n_assign(d) * size_t(d->d) * 2 < (size_t(1) << 31);
}
bool fuse_gather(const moe_desc* d) {
  return !gather_blocked(d) && size_t(d->T) * size_t(d->d) * act_bytes(d) < (size_t(1) << 31);
}
// With the fused gather on the prefill kernel in bf16, the layer first copies
// x into K-blocked planes in token order ([d/64][T][64]); the gate-up GEMM
// reads its routed rows from them through perm_token and the shared
// segment's rows in order.  The copy is x-sized (not T*k*d like x_perm), so
// it stays in the Infinity Cache.  With 32-column planes (DeepSeek-V3-shaped
// prefill: gate-up 8314 -> 7557 us for a 77 us copy) a row's piece of a plane
// was half a cache line: a tile's rows are an expert's tokens in increasing
// order, so neighbouring rows share a line only when both tokens chose the
// expert (78% of the bytes fetched were used on that layer, 72% on the
// Qwen-shaped one).  With 64-column planes (d is a multiple of 128) each
// piece is a whole 128-byte line, and the gate-up GEMM loads two stages' A
// per load.
bool x_blocked(const moe_desc* d) {
  return d->act == MOE_BF16 && !d->dispatch_fp8 && fuse_gather(d) && block_m(d) == 256;
}

// The layer's h between the routed GEMMs in K-blocked planes (GemmArgs::c_blk
// then a_blk): when the prefill kernel runs both in bf16, so each stage of the
// down projection reads one contiguous run per 32-column slice.  The matrices
// stay under 2^31 bytes, the reach of the kernel's 32-bit buffer offsets.
bool h_blocked(const moe_desc* d) {
  if (d->act != MOE_BF16 || block_m(d) != 256) return false;
  const size_t lim = size_t(1) << 31;
  return n_assign(d) * size_t(d->f) * 2 < lim && (!fuse_shared(d) || size_t(d->T) * d->f_shared * 2 < lim);
}
LayerWs carve_layer(Carve& c, const moe_desc* d) {
  LayerWs w;
  const size_t A = n_assign(d), ab = act_bytes(d);
  w.route = carve_route(c, d, reroute(d));
  w.disp = carve_dispatch(c, d, reroute(d));
  w.ffn = carve_ffn(c, d, fuse_shared(d));
  w.perm_token = c.take<int32_t>(sizeof(int32_t) * A);
  w.inv_pos = c.take<int32_t>(sizeof(int32_t) * A);
  w.offsets = c.take<int32_t>(sizeof(int32_t) * (d->E + 1));
  const size_t T = size_t(d->T);
  w.x_perm = fuse_gather(d) ? nullptr
                            : c.take<char>(d->dispatch_fp8 ? std::max(A * d->d * 2, payload_bytes(d, A))
                                                           : A * d->d * ab);
  w.xq = fuse_gather(d) && d->dispatch_fp8 ? c.take<char>(std::max(T * d->d * 2, payload_bytes(d, T))) : nullptr;
  w.xb = x_blocked(d) ? c.take<char>(T * d->d * 2) : nullptr;
  w.h = c.take<char>(A * d->f * ab);
  w.y_perm = c.take<char>(A * d->d * ab);
  w.sh = d->f_shared ? c.take<char>(size_t(d->T) * d->f_shared * ab) : nullptr;
  w.sy = d->f_shared ? c.take<char>(size_t(d->T) * d->d * ab) : nullptr;
  return w;
}

// moe_grouped_ffn given a payload that the gate-up GEMM cannot take as fp8:
// its values as bf16 rows.
void* carve_ffn_xdq(Carve& c, const moe_desc* d) {
  return d->dispatch_fp8 && !fp8_act(d) ? c.take<char>(size_t(n_assign(d)) * d->d * 2) : nullptr;
}

size_t stage_bytes(const moe_desc* d, moe_stage stage) {
  Carve c(nullptr);
  switch (stage) {
    case MOE_STAGE_ROUTE: carve_route(c, d, false); break;
    case MOE_STAGE_DISPATCH: carve_dispatch(c, d, reroute(d)); break;
    case MOE_STAGE_FFN:
      carve_ffn(c, d, false);
      carve_ffn_xdq(c, d);
      break;
    default: carve_layer(c, d); break;
  }
  return c.used;
}

moe_status dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

#define MOE_TRY(expr)                     \
  do {                                    \
    moe_status st_ = (expr);              \
    if (st_ != MOE_OK) return st_;        \
  } while (0)

// ---------------------------------------------------------------- stages
moe_status run_route(const moe_desc* d, const void* x, const void* wr, const float* bias,
                     int32_t* idx, float* w, const RouteWs& ws, hipStream_t s) {
  if (router_fused_ok(d->T, d->d, d->E, d->k, d->n_group, gemm_dtype(d->act))) {
    RouterFusedArgs r{x, wr, bias, d->T, d->d, d->E, d->k, d->score, d->renorm, idx, w, ws.cand_idx, ws.cand_w};
    return dev(launch_router_fused(r, s));
  }
  GemmArgs g{};
  g.A = x;
  g.rows = d->T;
  g.B0 = wr;
  g.bias = bias;
  g.N = d->E;
  g.K = d->d;
  g.C = ws.z;
  g.act = gemm_dtype(d->act);
  g.wdt = gemm_dtype(d->act);
  g.epi = EPI_BIAS_F32;
  g.ksplit = ws.ksplit;
  g.m_tile = big_router_plan(d).rows;  // used by the prefill kernel only
  MOE_TRY(dev(launch_gemm(g, s)));
  RouteSelectArgs r{ws.z, ws.ksplit, d->T, d->E, d->k, d->score, d->renorm, d->n_group, d->topk_group,
                    idx, w, ws.cand_idx, ws.cand_w};
  return dev(launch_route_select(r, s));
}

// rr: the rerouting dispatch's inputs (router gates and candidates) and
// workspace, or NULL for the dispatch of section "Dispatch" of moe.h.
moe_status run_dispatch(const moe_desc* d, const int32_t* idx, const void* x, int32_t* counts,
                        int32_t* offsets, int32_t* perm_token, int32_t* inv_pos, void* x_perm,
                        const DispatchWs& ws, hipStream_t s, const RerouteArgs* rr = nullptr,
                        bool blocked = false) {
  DispatchArgs a{idx, int(n_assign(d)), d->E, d->k, ws.chunk_cnt, counts, offsets, perm_token, inv_pos,
                 d->capacity > 0 ? d->capacity : INT32_MAX};
  MOE_TRY(dev(rr ? launch_dispatch_reroute(a, *rr, s) : launch_dispatch_index(a, s)));
  if (x_perm == nullptr) return MOE_OK;  // fused gather: GEMM1 reads x through perm_token
  // the gather stops at offsets[E] (the rows kept), read on the device
  if (blocked) return dev(launch_gather_rows_blocked(x, perm_token, int(n_assign(d)), offsets + d->E, d->d, 32, x_perm, s));
  return dev(launch_gather_rows(x, perm_token, int(n_assign(d)), offsets + d->E, int(d->d * act_bytes(d)),
                                x_perm, s));
}

// The fp8 payload of R rows of x into out: rows x[perm[p]] (perm NULL: in
// order) for p < min(R, *rows_dev); as codes + scales, or (values) as bf16.
moe_status run_payload(const moe_desc* d, const void* x, const int32_t* perm, int R, const int32_t* rows_dev,
                       bool values, void* out, hipStream_t s) {
  Fp8PayloadArgs p{};
  p.x = x;
  p.perm = perm;
  p.rows = R;
  p.rows_dev = rows_dev;
  p.d = d->d;
  p.sstride = int(payload_sstride(d));
  if (values) {
    p.deq = out;
  } else {
    p.codes = static_cast<uint8_t*>(out);
    p.scales = payload_scales(out, d, size_t(R));
  }
  return dev(launch_fp8_payload(p, s));
}

// Optional shared-expert segment of the routed launches (see fuse_shared).
struct SharedSeg {
  const void* x = nullptr;  // GEMM1 input: the tokens in order
  const void* w1 = nullptr;
  const void* w3 = nullptr;
  const void* w2 = nullptr;
  void* h = nullptr;        // GEMM1 output / GEMM2 input
  void* y = nullptr;        // GEMM2 output
};

// a_map: NULL (A = x_perm) or perm_token (A = x, the fused dispatch gather).
// a_scales: NULL (A in the act dtype) or the scales of a payload A (codes).
moe_status run_ffn_gemm1(const moe_desc* d, const void* A, const int32_t* a_map, const int32_t* offsets,
                         const void* w1, const void* w3, const float* s1, const float* s3, void* h,
                         const FfnWs& ws, hipStream_t s, const SharedSeg* sh = nullptr,
                         const uint8_t* a_scales = nullptr, bool h_blk = false, int a_blk = 0,
                         int sh_a_blk = 0) {
  GemmArgs g{};
  g.b_blk = d->w_layout == MOE_W_KBLOCKED;
  g.a_blk = a_blk;
  g.sh_a_blk = sh_a_blk;
  g.c_blk = h_blk;
  g.a_scales = a_scales;
  g.a_sstride = a_scales ? int(payload_sstride(d)) : 0;
  g.ksplit = 1;
  if (sh) {
    g.sh_rows = d->T;
    g.shA = sh->x;
    g.shB0 = sh->w1;
    g.shB1 = sh->w3;
    g.shC = sh->h;
    g.shN = d->f_shared;
    g.shK = d->d;
  }
  g.A = A;
  g.a_map = a_map;
  g.a_map_rows = a_map ? d->T : 0;
  g.rows = int(n_assign(d));
  g.E = d->E;
  g.tile_table = ws.table;
  g.offsets = offsets;
  g.n_slots = ws.n_slots;
  g.partial = ws.partial;
  g.partial_slots = ws.partial_slots;
  g.sched = ws.sched;
  g.sched_cap = ws.sched_cap;
  g.B0 = w1;
  g.B1 = w3;
  g.s0 = s1;
  g.s1 = s3;
  g.N = d->f;
  g.K = d->d;
  g.C = h;
  g.act = a_scales ? GD_FP8 : gemm_dtype(d->act);
  g.wdt = gemm_dtype(d->wdtype);
  g.epi = EPI_SWIGLU;
  return dev(launch_gemm(g, s));
}

moe_status run_ffn_gemm2(const moe_desc* d, const void* h, const int32_t* offsets, const void* w2,
                         const float* s2, void* y, const FfnWs& ws, hipStream_t s,
                         const SharedSeg* sh = nullptr, bool h_blk = false) {
  GemmArgs g{};
  g.b_blk = d->w_layout == MOE_W_KBLOCKED;
  g.a_blk = h_blk;
  g.sh_a_blk = h_blk;
  g.ksplit = 1;
  if (sh) {
    g.sh_rows = d->T;
    g.shA = sh->h;
    g.shB0 = sh->w2;
    g.shC = sh->y;
    g.shN = d->d;
    g.shK = d->f_shared;
  }
  g.A = h;
  g.rows = int(n_assign(d));
  g.E = d->E;
  g.tile_table = ws.table;
  g.offsets = offsets;
  g.n_slots = ws.n_slots;
  g.partial = ws.partial;
  g.partial_slots = ws.partial_slots;
  g.sched = ws.sched;
  g.sched_cap = ws.sched_cap;
  g.B0 = w2;
  g.s0 = s2;
  g.N = d->d;
  g.K = d->f;
  g.C = y;
  g.act = gemm_dtype(d->act);
  g.wdt = gemm_dtype(d->wdtype);
  g.epi = EPI_STORE;
  return dev(launch_gemm(g, s));
}

moe_status run_tables(const moe_desc* d, const int32_t* offsets, const FfnWs& ws, hipStream_t s,
                      bool with_shared = false) {
  TileTableArgs t{offsets, d->E, with_shared ? d->T : 0, block_m(d), ws.n_slots, ws.table, 0, 0,
                  nullptr};
  return dev(launch_tile_tables(t, s));
}

moe_status run_shared(const moe_desc* d, const void* x, const void* sw1, const void* sw3,
                      const void* sw2, void* sh, void* sy, hipStream_t s) {
  GemmArgs g{};
  g.ksplit = 1;
  g.A = x;
  g.rows = d->T;
  g.B0 = sw1;
  g.B1 = sw3;
  g.N = d->f_shared;
  g.K = d->d;
  g.C = sh;
  g.act = gemm_dtype(d->act);
  g.wdt = gemm_dtype(d->act);
  g.epi = EPI_SWIGLU;
  MOE_TRY(dev(launch_gemm(g, s)));
  GemmArgs g2{};
  g2.ksplit = 1;
  g2.A = sh;
  g2.rows = d->T;
  g2.B0 = sw2;
  g2.N = d->d;
  g2.K = d->f_shared;
  g2.C = sy;
  g2.act = gemm_dtype(d->act);
  g2.wdt = gemm_dtype(d->act);
  g2.epi = EPI_STORE;
  return dev(launch_gemm(g2, s));
}

bool fp8(const moe_desc* d) { return d->wdtype == MOE_FP8_E4M3; }

// scales must be present exactly when the weights are fp8
bool scales_ok(const moe_desc* d, const float* s1, const float* s3, const float* s2) {
  if (fp8(d)) return need(s1) && need(s3) && need(s2);
  return s1 == nullptr && s3 == nullptr && s2 == nullptr;
}

// The current device's copy of `scratch`, looked up on the first call on
// that device (with the device current) and kept: MOE_ERR_DEVICE if the
// lookup fails.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::array<void*, kMaxDevices> g_scratch_ptr{};
moe_status scratch_on_current_device(void** out) {
  int dev_id = -1;
  if (hipGetDevice(&dev_id) != hipSuccess) return MOE_ERR_DEVICE;
  if (dev_id < 0 || dev_id >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev_id] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_DEVICE;
    g_scratch_ptr[dev_id] = p;
  }
  *out = g_scratch_ptr[dev_id];
  return MOE_OK;
}

// moe_dispatch after validation, on a workspace of at least
// stage_bytes(d, MOE_STAGE_DISPATCH) bytes.
moe_status dispatch_on(const moe_desc* d, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* perm_token, int32_t* inv_pos, void* x_perm, void* ws,
                       hipStream_t s) {
  Carve c(ws);
  const DispatchWs w = carve_dispatch(c, d, false);
  if (!d->dispatch_fp8)
    return run_dispatch(d, topk_idx, x, counts, offsets, perm_token, inv_pos, x_perm, w, s);
  MOE_TRY(run_dispatch(d, topk_idx, x, counts, offsets, perm_token, inv_pos, nullptr, w, s));
  if (d->T == 0) return MOE_OK;
  return run_payload(d, x, perm_token, int(n_assign(d)), offsets + d->E, false, x_perm, s);
}

moe_status record(void* const* trace, int i, hipStream_t s) {
  if (trace == nullptr) return MOE_OK;
  return dev(hipEventRecord(static_cast<hipEvent_t>(trace[i]), s));
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or dtype not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: HIP call or kernel launch failed";
  }
  return "unknown moe_status";
}

moe_status moe_validate(const moe_desc* desc) { return check_desc(desc); }

moe_status moe_capacity_slots(int64_t factor_num, int64_t factor_den, int32_t T, int32_t k, int32_t E,
                              int32_t* slots) {
  if (slots == nullptr || factor_den <= 0 || T < 0 || k < 1 || E < 1) return MOE_ERR_INVALID;
  if (factor_num <= 0) {
    *slots = 0;
    return MOE_OK;
  }
  // ceil(num * T * k / (den * E)), exact in 128 bits: num < 2^63, T, k < 2^31
  const unsigned __int128 num = (unsigned __int128)uint64_t(factor_num) * uint32_t(T) * uint32_t(k);
  const unsigned __int128 den = (unsigned __int128)uint64_t(factor_den) * uint32_t(E);
  const unsigned __int128 q = (num + den - 1) / den;
  if (q > (unsigned __int128)INT32_MAX) return MOE_ERR_INVALID;
  *slots = int32_t(q);
  return MOE_OK;
}

moe_status moe_pack_weights(const void* src, int64_t mats, int32_t rows, int32_t cols, int32_t elem_bytes,
                            void* dst, void* stream) {
  if (mats < 0 || rows < 0 || cols < 0 || cols % 32 != 0 || (elem_bytes != 1 && elem_bytes != 2))
    return MOE_ERR_INVALID;
  const unsigned __int128 wide = (unsigned __int128)mats * uint32_t(rows) * uint32_t(cols) * uint32_t(elem_bytes);
  if (wide > ((unsigned __int128)1 << 40)) return MOE_ERR_INVALID;
  const int64_t bytes = int64_t(wide);
  if (bytes == 0) return MOE_OK;
  if (!need(src) || !need(dst)) return MOE_ERR_INVALID;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + uint64_t(bytes) && d0 < s0 + uint64_t(bytes)) return MOE_ERR_INVALID;  // overlap
  return dev(launch_pack_kblocked(src, mats, rows, cols, elem_bytes, dst, static_cast<hipStream_t>(stream)));
}

moe_status moe_workspace_size(const moe_desc* desc, moe_stage stage, size_t* bytes) {
  MOE_TRY(check_desc(desc));
  if (bytes == nullptr) return MOE_ERR_INVALID;
  if (stage < MOE_STAGE_ROUTE || stage > MOE_STAGE_LAYER) return MOE_ERR_INVALID;
  *bytes = stage_bytes(desc, stage);
  return MOE_OK;
}

moe_status moe_route(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(d));
  if (d->T == 0) return MOE_OK;
  if (!need(x) || !need(w_router) || !maybe(bias) || !need(topk_idx) || !need(topk_w) || !need(ws))
    return MOE_ERR_INVALID;
  if (ws_bytes < stage_bytes(d, MOE_STAGE_ROUTE)) return MOE_ERR_WORKSPACE;
  Carve c(ws);
  const RouteWs w = carve_route(c, d, false);
  return run_route(d, x, w_router, bias, topk_idx, topk_w, w, static_cast<hipStream_t>(stream));
}

moe_status moe_route_candidates(const moe_desc* d, const void* x, const void* w_router, const float* bias,
                                int32_t* topk_idx, float* topk_w, int32_t* cand_idx, float* cand_w, void* ws,
                                size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(d));
  if (d->T == 0) return MOE_OK;
  if (!need(x) || !need(w_router) || !maybe(bias) || !need(topk_idx) || !need(topk_w) || !need(cand_idx) ||
      !need(cand_w) || !need(ws))
    return MOE_ERR_INVALID;
  if (ws_bytes < stage_bytes(d, MOE_STAGE_ROUTE)) return MOE_ERR_WORKSPACE;
  Carve c(ws);
  RouteWs w = carve_route(c, d, false);
  w.cand_idx = cand_idx;
  w.cand_w = cand_w;
  return run_route(d, x, w_router, bias, topk_idx, topk_w, w, static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch_reroute(const moe_desc* d, const int32_t* topk_idx, const float* topk_w,
                                const int32_t* cand_idx, const float* cand_w, const void* x, int32_t* counts,
                                int32_t* offsets, int32_t* perm_token, int32_t* inv_pos, float* gates,
                                void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(d));
  if (!reroute(d)) return MOE_ERR_INVALID;
  if (!need(counts) || !need(offsets)) return MOE_ERR_INVALID;
  if (d->T > 0 && (!need(topk_idx) || !need(topk_w) || !need(cand_idx) || !need(cand_w) || !need(x) ||
                   !need(perm_token) || !need(inv_pos) || !need(gates) || !need(x_perm) || !need(ws)))
    return MOE_ERR_INVALID;
  if (d->T > 0 && ws_bytes < stage_bytes(d, MOE_STAGE_DISPATCH)) return MOE_ERR_WORKSPACE;
  Carve c(ws);
  const DispatchWs w = carve_dispatch(c, d, true);
  RerouteArgs rr = w.rr;
  rr.topk_w = topk_w;
  rr.cand_idx = cand_idx;
  rr.cand_w = cand_w;
  rr.gate = gates;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(run_dispatch(d, topk_idx, x, counts, offsets, perm_token, inv_pos, d->dispatch_fp8 ? nullptr : x_perm,
                       w, s, &rr));
  if (d->T == 0 || !d->dispatch_fp8) return MOE_OK;
  return run_payload(d, x, perm_token, int(n_assign(d)), offsets + d->E, false, x_perm, s);
}

moe_status moe_dispatch(const moe_desc* d, const int32_t* topk_idx, const void* x, int32_t* counts,
                        int32_t* offsets, int32_t* perm_token, int32_t* inv_pos, void* x_perm,
                        void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(d));
  if (reroute(d)) return MOE_ERR_UNSUPPORTED;  // needs the router's candidates: moe_layer_forward only
  if (!need(counts) || !need(offsets)) return MOE_ERR_INVALID;
  if (d->T > 0 && (!need(topk_idx) || !need(x) || !need(perm_token) || !need(inv_pos) ||
                   !need(x_perm) || !need(ws)))
    return MOE_ERR_INVALID;
  if (d->T > 0 && ws_bytes < stage_bytes(d, MOE_STAGE_DISPATCH)) return MOE_ERR_WORKSPACE;
  return dispatch_on(d, topk_idx, x, counts, offsets, perm_token, inv_pos, x_perm, ws,
                     static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch_noalloc(const moe_desc* d, const int32_t* topk_idx, const void* x, int32_t* counts,
                                int32_t* offsets, int32_t* perm_token, int32_t* inv_pos, void* x_perm,
                                void* stream) {
  MOE_TRY(check_desc(d));
  if (reroute(d)) return MOE_ERR_UNSUPPORTED;  // as moe_dispatch
  if (!need(counts) || !need(offsets)) return MOE_ERR_INVALID;
  if (d->T > 0 && (!need(topk_idx) || !need(x) || !need(perm_token) || !need(inv_pos) || !need(x_perm)))
    return MOE_ERR_INVALID;
  if (stage_bytes(d, MOE_STAGE_DISPATCH) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  MOE_TRY(scratch_on_current_device(&ws));
  return dispatch_on(d, topk_idx, x, counts, offsets, perm_token, inv_pos, x_perm, ws,
                     static_cast<hipStream_t>(stream));
}

moe_status moe_grouped_ffn(const moe_desc* d, const void* x_perm, const int32_t* offsets,
                           const void* w1, const void* w3, const void* w2, const float* s1,
                           const float* s3, const float* s2, void* h, void* y_perm, void* ws,
                           size_t ws_bytes, void* stream) {
  MOE_TRY(check_desc(d));
  if (d->T == 0) return MOE_OK;
  if (!need(x_perm) || !need(offsets) || !need(w1) || !need(w3) || !need(w2) || !need(h) ||
      !need(y_perm) || !need(ws) || !scales_ok(d, s1, s3, s2))
    return MOE_ERR_INVALID;
  if (ws_bytes < stage_bytes(d, MOE_STAGE_FFN)) return MOE_ERR_WORKSPACE;
  Carve c(ws);
  const FfnWs w = carve_ffn(c, d, false);
  void* xdq = carve_ffn_xdq(c, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(run_tables(d, offsets, w, s));
  const size_t A = size_t(n_assign(d));
  if (d->dispatch_fp8 && fp8_act(d)) {
    MOE_TRY(run_ffn_gemm1(d, x_perm, nullptr, offsets, w1, w3, s1, s3, h, w, s, nullptr,
                          payload_scales(const_cast<void*>(x_perm), d, A)));
  } else if (d->dispatch_fp8) {
    const uint8_t* codes = static_cast<const uint8_t*>(x_perm);
    MOE_TRY(dev(launch_fp8_dequant(codes, payload_scales(const_cast<void*>(x_perm), d, A), int(payload_sstride(d)),
                                   int(A), offsets + d->E, d->d, xdq, s)));
    MOE_TRY(run_ffn_gemm1(d, xdq, nullptr, offsets, w1, w3, s1, s3, h, w, s));
  } else {
    MOE_TRY(run_ffn_gemm1(d, x_perm, nullptr, offsets, w1, w3, s1, s3, h, w, s));
  }
  return run_ffn_gemm2(d, h, offsets, w2, s2, y_perm, w, s);
}

moe_status moe_combine(const moe_desc* d, const void* y_perm, const int32_t* inv_pos,
                       const float* topk_w, const void* shared_y, void* out, void* stream) {
  MOE_TRY(check_desc(d));
  if (d->T == 0) return MOE_OK;
  if (!need(y_perm) || !need(inv_pos) || !need(topk_w) || !maybe(shared_y) || !need(out))
    return MOE_ERR_INVALID;
  CombineArgs a{y_perm, inv_pos, topk_w, shared_y, out, d->T, d->d, d->k, gemm_dtype(d->act)};
  return dev(launch_combine(a, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(const moe_desc* d, const void* x, const void* w_router,
                             const float* bias, const void* w1, const void* w3, const void* w2,
                             const float* s1, const float* s3, const float* s2, const void* sw1,
                             const void* sw3, const void* sw2, void* out, int32_t* topk_idx,
                             float* topk_w, int32_t* counts, void* ws, size_t ws_bytes,
                             void* stream, void* const* trace) {
  MOE_TRY(check_desc(d));
  if (!need(counts)) return MOE_ERR_INVALID;
  const bool shared = d->f_shared > 0;
  if (d->T > 0) {
    if (!need(x) || !need(w_router) || !maybe(bias) || !need(w1) || !need(w3) || !need(w2) ||
        !scales_ok(d, s1, s3, s2) || !need(out) || !need(topk_idx) || !need(topk_w) || !need(ws))
      return MOE_ERR_INVALID;
    if (shared ? !(need(sw1) && need(sw3) && need(sw2)) : (sw1 || sw3 || sw2))
      return MOE_ERR_INVALID;
  }
  if (d->T > 0 && (ws_bytes < stage_bytes(d, MOE_STAGE_LAYER) || ws == nullptr))
    return MOE_ERR_WORKSPACE;
  if (trace) {
    for (int i = 0; i < MOE_TRACE_EVENTS; ++i)
      if (trace[i] == nullptr) return MOE_ERR_INVALID;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->T == 0) {  // nothing routed: counts are all zero
    DispatchArgs a{nullptr, 0, d->E, d->k, nullptr, counts, nullptr, nullptr, nullptr, INT32_MAX};
    return dev(launch_dispatch_index(a, s));
  }
  Carve c(ws);
  const LayerWs w = carve_layer(c, d);
  MOE_TRY(record(trace, 0, s));
  MOE_TRY(run_route(d, x, w_router, bias, topk_idx, topk_w, w.route, s));
  MOE_TRY(record(trace, 1, s));
  const bool fg = fuse_gather(d);  // GEMM1 reads its rows through perm_token
  const bool gb = gather_blocked(d);  // or from x_perm in K-blocked planes
  RerouteArgs rr = w.disp.rr;
  rr.topk_w = topk_w;
  rr.cand_idx = w.route.cand_idx;
  rr.cand_w = w.route.cand_w;
  MOE_TRY(run_dispatch(d, topk_idx, x, counts, w.offsets, w.perm_token, w.inv_pos,
                       d->dispatch_fp8 ? nullptr : w.x_perm, w.disp, s, reroute(d) ? &rr : nullptr, gb));
  // GEMM1's activation rows: x, the gathered x_perm, or the fp8 payload (in
  // token order when the gather is fused, else gathered), as codes when the
  // GEMM takes fp8 activations, else as bf16 values
  const bool xb = x_blocked(d);
  if (xb) MOE_TRY(dev(launch_gather_rows_blocked(x, nullptr, d->T, nullptr, d->d, 64, w.xb, s)));
  const void* a_rows = xb ? w.xb : fg ? x : w.x_perm;
  const uint8_t* a_scales = nullptr;
  if (d->dispatch_fp8) {
    const bool f8 = fp8_act(d);
    const int R = fg ? d->T : int(n_assign(d));
    void* dst = fg ? w.xq : w.x_perm;
    MOE_TRY(run_payload(d, x, fg ? nullptr : w.perm_token, R, fg ? nullptr : w.offsets + d->E, !f8, dst, s));
    a_rows = dst;
    if (f8) a_scales = payload_scales(dst, d, size_t(R));
  }
  const bool fused = fuse_shared(d);
  SharedSeg sh;
  if (fused) {
    sh.x = xb ? w.xb : x;
    sh.w1 = sw1;
    sh.w3 = sw3;
    sh.w2 = sw2;
    sh.h = w.sh;
    sh.y = w.sy;
  }
  MOE_TRY(run_tables(d, w.offsets, w.ffn, s, fused));
  const bool hb = h_blocked(d);
  MOE_TRY(record(trace, 2, s));
  // A (and the shared segment's x) K-blocked: 64-column planes for the copy
  // of x, 32 for the gathered x_perm
  const int ablk = xb ? 2 : gb ? 1 : 0;
  MOE_TRY(run_ffn_gemm1(d, a_rows, fg ? w.perm_token : nullptr, w.offsets, w1, w3, s1, s3, w.h, w.ffn, s,
                        fused ? &sh : nullptr, a_scales, hb, ablk, xb ? ablk : 0));
  MOE_TRY(record(trace, 3, s));
  MOE_TRY(run_ffn_gemm2(d, w.h, w.offsets, w2, s2, w.y_perm, w.ffn, s, fused ? &sh : nullptr, hb));
  MOE_TRY(record(trace, 4, s));
  if (shared && !fused) MOE_TRY(run_shared(d, x, sw1, sw3, sw2, w.sh, w.sy, s));
  MOE_TRY(record(trace, 5, s));
  // a rerouted copy carries its new expert's gate
  CombineArgs a{w.y_perm, w.inv_pos, reroute(d) ? rr.gate : topk_w, shared ? w.sy : nullptr, out, d->T, d->d,
                d->k, gemm_dtype(d->act)};
  MOE_TRY(dev(launch_combine(a, s)));
  return record(trace, 6, s);
}

moe_status moe_layer_rows(const moe_desc* d, const void* ws, size_t ws_bytes, int32_t* rows, void* stream) {
  MOE_TRY(check_desc(d));
  if (!need(rows)) return MOE_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->T == 0) {  // moe_layer_forward laid out no rows
    DispatchArgs a{nullptr, 0, d->E, d->k, nullptr, rows, nullptr, nullptr, nullptr, INT32_MAX};
    return dev(launch_dispatch_index(a, s));
  }
  if (!need(ws)) return MOE_ERR_INVALID;
  if (ws_bytes < stage_bytes(d, MOE_STAGE_LAYER)) return MOE_ERR_WORKSPACE;
  Carve c(const_cast<void*>(ws));
  const LayerWs w = carve_layer(c, d);
  return dev(launch_segment_rows(w.offsets, d->E, rows, s));
}

}  // extern "C"
