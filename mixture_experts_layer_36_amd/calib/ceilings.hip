// Ceiling probes for the bench's roofline figures, kept apart from the layer
// library (libmoe_calib.so, loaded only by bench.py).  Each measures what one
// gfx950 unit sustains with nothing else in the way:
//   * the MFMA pattern of a prefill GEMM stage on its own: one wavefront per
//     SIMD (one block of four per CU), operands from two alternating
//     register sets; bf16 as the bf16-operand tiles run it
//     (v_mfma_f32_16x16x32_bf16 on an 8 x 4 grid of 16x16 accumulators, 8
//     weight and 4 activation fragments per set), fp8 as the fp8 x fp8
//     tiles do (v_mfma_scale_f32_32x32x64_f8f6f4 on a 4 x 4 grid of 32x32
//     accumulators); with random operand values (the MFMA's power, and so
//     the clock the chip holds, depends on how the operand bits toggle: a
//     loop on constant operands runs at full clock, one on random data does
//     not) or constant ones.  Both do 32 x 32768 flops per wavefront and
//     iteration;
//   * a streaming read: each block reads one contiguous chunk with 16-byte
//     loads, consecutive lanes on consecutive 16-byte pieces, with plain or
//     non-temporal loads.
// Results are folded into one value per thread and stored only if it equals
// a value the inputs cannot produce, so nothing is optimised away and the
// probes write (almost) nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 c_bf16x8 __attribute__((ext_vector_type(8)));
typedef float c_f32x16 __attribute__((ext_vector_type(16)));
typedef float c_f32x4 __attribute__((ext_vector_type(4)));
typedef int c_i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t c_u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;

// A 32-bit mix of the thread and register index (the "lowbias32" integer
// hash): the operand values of the GEMM-shaped probes.
__device__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 operands: random values in [-2, 2) unless `constant`.
__global__ __launch_bounds__(kThreads, 1) void mfma_bf16_gemm_shape(int iters, int constant, float* sink) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  c_bf16x8 w[2][8], x[2][4];
  for (int s = 0; s < 2; ++s)
    for (int q = 0; q < 8; ++q)
      for (int i = 0; i < 8; ++i) {
        const uint32_t r = mix32(t * 977u + s * 131u + q * 17u + i + 1u);
        w[s][q][i] = (__bf16)(constant ? 1.0f : float(int(r & 0xffff) - 32768) / 16384.0f);
        if (q < 4) x[s][q][i] = (__bf16)(constant ? 0.5f : float(int(r >> 16) - 32768) / 16384.0f);
      }
  c_f32x4 acc[8][4];
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j)
      for (int q = 0; q < 4; ++q) acc[i][j][q] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[s][i], x[s][j], acc[i][j], 0, 0, 0);
  }
  float v = 0.0f;
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j)
      for (int q = 0; q < 4; ++q) v += acc[i][j][q];
  if (v == -1.2345e-30f) sink[t] = v;
}

// fp8 operands: random finite E4M3 codes (a NaN code 0x7f / 0xff becomes
// 0x7e / 0xfe) unless `constant`; unit block scales.
__global__ __launch_bounds__(kThreads, 1) void mfma_fp8_gemm_shape(int iters, int constant, float* sink) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  c_i32x8 w[2][4], x[2][4];
  auto code4 = [&](uint32_t r) {
    uint32_t o = 0;
    for (int b = 0; b < 4; ++b) {
      uint32_t c = (r >> (8 * b)) & 0xffu;
      if ((c & 0x7fu) == 0x7fu) c ^= 1u;
      o |= c << (8 * b);
    }
    return int(o);
  };
  for (int s = 0; s < 2; ++s)
    for (int q = 0; q < 4; ++q)
      for (int i = 0; i < 8; ++i) {
        w[s][q][i] = constant ? int(0x38383838u) : code4(mix32(t * 977u + s * 131u + q * 17u + i + 1u));
        x[s][q][i] = constant ? int(0x30303030u) : code4(mix32(t * 1009u + s * 137u + q * 19u + i + 7u));
      }
  c_f32x16 acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w[s][i], x[s][j], acc[i][j], 0, 0, 0, 127, 0, 127);
  }
  float v = 0.0f;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      for (int q = 0; q < 16; ++q) v += acc[i][j][q];
  if (v == -1.2345e-30f) sink[t] = v;
}

// Block b reads bytes [b * chunk, (b + 1) * chunk); chunk is a multiple of
// 16 * kThreads * kUnroll, so every 16-byte load of the block lies inside its
// chunk.  Each thread keeps kUnroll loads in flight.  NT: non-temporal loads
// (the nt bit; on MI355X a stream read this way is ~13% faster).
constexpr int kUnroll = 8;
template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read(const c_u32x4* src, long long chunk16, uint32_t* sink) {
  const c_u32x4* p = src + (long long)blockIdx.x * chunk16 + threadIdx.x;
  c_u32x4 x = {0u, 0u, 0u, 0u};
  for (long long i = 0; i < chunk16; i += kThreads * kUnroll) {
    c_u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = NT ? __builtin_nontemporal_load(&p[i + u * kThreads]) : p[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u];
  }
  const uint32_t v = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (v == 0x9e3779b9u) sink[blockIdx.x * kThreads + threadIdx.x] = v;
}

}  // namespace

extern "C" {

// GEMM-shaped probes.  flop of one launch: blocks * 4 wavefronts * iters *
// 32 MFMAs * (32*32*16*2 for bf16, 32*32*64*2 for fp8); constant != 0 runs
// constant operands, else random ones.  sink: device, blocks * 256 floats.
int moe_calib_mfma_bf16_gemm(int blocks, int iters, int constant, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || sink == nullptr) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_bf16_gemm_shape, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                     constant, sink);
  return int(hipGetLastError());
}
int moe_calib_mfma_fp8_gemm(int blocks, int iters, int constant, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || sink == nullptr) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_fp8_gemm_shape, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                     constant, sink);
  return int(hipGetLastError());
}

// Reads blocks * chunk bytes of src, chunk = floor(bytes / blocks) rounded
// down to a multiple of 32768; returns that byte count in *read (host).
// src 16-byte aligned; sink: device, blocks * 256 uint32; nt != 0: with
// non-temporal loads.
int moe_calib_stream_read(const void* src, long long bytes, int blocks, uint32_t* sink, long long* read,
                          int nt, void* stream) {
  if (src == nullptr || sink == nullptr || read == nullptr || blocks <= 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return int(hipErrorInvalidValue);
  const long long unit = 16LL * kThreads * kUnroll;
  const long long chunk = bytes / blocks / unit * unit;
  if (chunk <= 0) return int(hipErrorInvalidValue);
  *read = chunk * blocks;
  if (nt)
    hipLaunchKernelGGL(stream_read<true>, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const c_u32x4*>(src), chunk / 16, sink);
  else
    hipLaunchKernelGGL(stream_read<false>, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const c_u32x4*>(src), chunk / 16, sink);
  return int(hipGetLastError());
}

}  // extern "C"
