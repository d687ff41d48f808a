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

// The scale comes from integer arithmetic on the bf16 bits of the block's
// largest magnitude.  Each element is scaled by 2^-s exactly (an exponent
// change; a bf16 subnormal goes through its integer significand, so no step
// depends on the float denormal mode) and converted by the hardware
// f32 -> E4M3 conversion, which rounds to nearest even with OCP subnormals
// (checked against a brute-force nearest search over a 2^-14 grid up to 16 and
// against the oracle's codes).  It gives -0 for a negative value that rounds
// to zero; the payload's zero is +0.

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
  // x * 2^-s as a float (exact: |x| * 2^-s <= 448; values that would leave
  // the normal range are far below half the smallest E4M3 step)
  auto scaled = [&](uint32_t b) -> float {
    const uint32_t mag = b & 0x7fffu;
    const float v = (mag >> 7) ? ldexpf(__uint_as_float(mag << 16), -s) : ldexpf((float)mag, -133 - s);
    return (b & 0x8000u) ? -v : v;
  };
  uint32_t codes[8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; q += 2) {  // elements 8i + 2q .. 8i + 2q + 3
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(v[i][q] & 0xffffu), scaled(v[i][q] >> 16), 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(v[i][q + 1] & 0xffffu), scaled(v[i][q + 1] >> 16), w, true);
      const uint32_t u = (uint32_t)w;
      const uint32_t nz = ((u & 0x7f7f7f7fu) + 0x7f7f7f7fu) & 0x80808080u;  // magnitude != 0, per byte
      codes[i * 2 + q / 2] = (u & 0x7f7f7f7fu) | (u & nz);                 // -0 -> +0
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
