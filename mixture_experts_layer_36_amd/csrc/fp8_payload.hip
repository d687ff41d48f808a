// The fp8 dispatch payload: token rows quantised to OCP E4M3 in blocks of 32
// elements, each block with one power-of-two scale (an E8M0 byte).
//
// DeepSeek's serving system sends the dispatch token copies in FP8 and the
// combine results in BF16 ("Tensor vs Expert vs Data Parallelism for MoE
// Serving", section "Deeper Analysis", Figure 2; section "What Goes Wrong",
// on precision and communication).  The block of 32 with a power-of-two
// scale is the format gfx950's block-scaled MFMA consumes directly: in
// v_mfma_scale_f32_32x32x64_f8f6f4 each lane supplies 32 consecutive k values
// of one row and one E8M0 scale for them.
//
// A block with largest magnitude amax takes the scale 2^s with s the smallest
// integer such that amax <= 448 * 2^s, so no element saturates; elements
// become E4M3 codes of x * 2^-s rounded to nearest, ties to even.  An
// all-zero block gets s = 0.
//
// Kernels (one thread per 32-element block):
//   * rows in order -> codes [rows][d] and scales [rows][sstride] (the layer's
//     fused path: the gate-up GEMM then reads them through perm_token);
//   * gathered rows x[perm[p]] -> the same layout (the dispatch entry point's
//     fp8 x_perm), rows p < *rows_dev;
//   * rows (in order or gathered) -> the dequantised payload as bf16 rows,
//     for GEMM paths without fp8 activations;
//   * codes + scales -> bf16 rows (the grouped FFN given a payload).
// A scaled E4M3 value is a bf16 value unless it falls below bf16's smallest
// subnormal (2^-133), which takes a block whose largest magnitude is under
// 2^-115; such values round to the nearest bf16.
#include "moe_internal.hpp"

namespace moe {
namespace {

// Everything is integer arithmetic on the bf16 bits, so subnormal inputs
// and scaled values are exact whatever the float denormal mode.
//
// E4M3 magnitude code of M * 2^q (M: an integer significand, 1..255; the
// value must be <= 448).  With e the value's binary exponent and eb =
// max(e, -6), the code's step is 2^(eb - 3) (normal codes hold 8..15 steps,
// subnormal ones 0..7 steps of 2^-9), so the code is (eb + 6) * 8 + r with r
// the value in steps rounded to nearest even; r = 16 (or 8 for a subnormal)
// lands exactly on the next binade's first code.
__device__ __forceinline__ uint32_t e4m3_code(uint32_t M, int q) {
  const int nb = 32 - __builtin_clz(M);  // bit length
  const int e = nb - 1 + q;
  const int eb = e < -6 ? -6 : e;
  const int shift = eb - 3 - q;
  uint32_t r;
  if (shift <= 0) {
    r = M << (-shift);
  } else if (shift > 9) {
    r = 0;  // below half a step (M < 2^8)
  } else {
    r = M >> shift;
    const uint32_t rem = M & ((1u << shift) - 1u), half = 1u << (shift - 1);
    r += (rem > half || (rem == half && (r & 1u))) ? 1u : 0u;
  }
  return r == 0 ? 0u : (uint32_t)((eb + 6) * 8) + r;
}

// bf16 magnitude bits (no sign) -> (M, q) with value M * 2^q, M >= 1.
__device__ __forceinline__ void bf16_sig(uint32_t mag, uint32_t& M, int& q) {
  const uint32_t ef = mag >> 7, m = mag & 0x7fu;
  if (ef == 0) {  // subnormal: m * 2^-133
    M = m;
    q = -133;
  } else {
    M = m | 0x80u;
    q = (int)ef - 134;  // (128 + m) * 2^(ef - 127 - 7)
  }
}

// Scale exponent s of a block whose largest magnitude has bf16 bits amag:
// with amax = (1 + m/128) * 2^e, the smallest s with amax <= 448 * 2^s =
// 1.75 * 2^(s + 8) is e - 8 when m <= 96 (1 + m/128 <= 1.75), else e - 7.
// Clamped to [-127, 127] (a subnormal amax always takes -127); 0 for zero.
__device__ __forceinline__ int block_scale_exp(uint32_t amag) {
  if (amag == 0) return 0;
  const int ef = (int)(amag >> 7);
  if (ef == 0) return -127;
  const int e = ef - 127;
  const int s = ((amag & 0x7fu) <= 96u) ? e - 8 : e - 7;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

__global__ __launch_bounds__(256) void fp8_payload_kernel(Fp8PayloadArgs a) {
  const int nb = a.d / 32;  // blocks per row
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int row = (int)(g / nb), blk = (int)(g % nb);
  const int rows = a.rows_dev ? min(*a.rows_dev, a.rows) : a.rows;
  if (row >= rows) return;
  const int src = a.perm ? a.perm[row] : row;
  const u32x4* xin = (const u32x4*)((const uint16_t*)a.x + (size_t)src * a.d + blk * 32);
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = xin[i];
  uint32_t amag = 0;  // magnitudes order like their bit patterns (no NaN/Inf in x)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amag = max(amag, v[i][q] & 0x7fffu);
      amag = max(amag, (v[i][q] >> 16) & 0x7fffu);
    }
  const int s = block_scale_exp(amag);
  uint32_t codes[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t b = h ? (v[i][q] >> 16) : (v[i][q] & 0xffffu);
        const uint32_t mag = b & 0x7fffu;
        uint32_t c = 0;
        if (mag != 0) {
          uint32_t M;
          int e2;
          bf16_sig(mag, M, e2);
          c = e4m3_code(M, e2 - s);
          if (c != 0) c |= (b & 0x8000u) ? 0x80u : 0u;
        }
        const int idx = (i * 4 + q) * 2 + h;  // element 0..31
        codes[idx >> 2] |= c << ((idx & 3) * 8);
      }
  if (a.deq) {  // dequantised bf16 payload
    u32x4* out = (u32x4*)((uint16_t*)a.deq + (size_t)row * a.d + blk * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = (i * 4 + q) * 2;
        const uint32_t c0 = (codes[idx >> 2] >> ((idx & 3) * 8)) & 0xffu;
        const uint32_t c1 = (codes[(idx + 1) >> 2] >> (((idx + 1) & 3) * 8)) & 0xffu;
        // E4M3 value as bf16 bits, then the power of two on the exponent
        const float f0 = ldexpf(bf16_to_f32(e4m3_to_bf16(c0)), s);
        const float f1 = ldexpf(bf16_to_f32(e4m3_to_bf16(c1)), s);
        o[q] = pack_bf16x2(f0, f1);
      }
      out[i] = o;
    }
    return;
  }
  u32x4* cout = (u32x4*)(a.codes + (size_t)row * a.d + blk * 32);
  cout[0] = u32x4{codes[0], codes[1], codes[2], codes[3]};
  cout[1] = u32x4{codes[4], codes[5], codes[6], codes[7]};
  a.scales[(size_t)row * a.sstride + blk] = (uint8_t)(s + 127);
}

__global__ __launch_bounds__(256) void fp8_dequant_kernel(const uint8_t* codes, const uint8_t* scales, int sstride,
                                                          int rows, const int32_t* rows_dev, int d, void* out) {
  const int nb = d / 32;
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int row = (int)(g / nb), blk = (int)(g % nb);
  const int n = rows_dev ? min(*rows_dev, rows) : rows;
  if (row >= n) return;
  const u32x4* cin = (const u32x4*)(codes + (size_t)row * d + blk * 32);
  const int s = (int)scales[(size_t)row * sstride + blk] - 127;
  u32x4* o = (u32x4*)((uint16_t*)out + (size_t)row * d + blk * 32);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 c = cin[i];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = c[half * 2 + q / 2] >> ((q & 1) * 16);
        const float f0 = ldexpf(bf16_to_f32(e4m3_to_bf16(w & 0xffu)), s);
        const float f1 = ldexpf(bf16_to_f32(e4m3_to_bf16((w >> 8) & 0xffu)), s);
        v[q] = pack_bf16x2(f0, f1);
      }
      o[i * 2 + half] = v;
    }
  }
}

}  // namespace

hipError_t launch_fp8_dequant(const uint8_t* codes, const uint8_t* scales, int sstride, int rows,
                              const int32_t* rows_dev, int d, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const size_t threads = (size_t)rows * (d / 32);
  hipLaunchKernelGGL(fp8_dequant_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, codes, scales,
                     sstride, rows, rows_dev, d, out);
  return hipGetLastError();
}

hipError_t launch_fp8_payload(const Fp8PayloadArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const size_t threads = (size_t)a.rows * (a.d / 32);
  hipLaunchKernelGGL(fp8_payload_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
