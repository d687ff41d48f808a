// Ceiling probes for the bench's roofline figures, kept apart from the layer
// library (libmoe_calib.so, loaded only by bench.py).  Each measures what one
// gfx950 unit sustains with nothing else in the way:
//   * a register-only loop of bf16 MFMAs (v_mfma_f32_32x32x16_bf16), four
//     independent accumulator chains per wavefront, four wavefronts per block;
//   * the same with the block-scaled fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4,
//     E4M3 operands, unit scales);
//   * a streaming read: each block reads one contiguous chunk with 16-byte
//     loads, consecutive lanes on consecutive 16-byte pieces.
// Results are folded into one value per thread and stored only if it equals
// a value the inputs cannot produce, so nothing is optimised away and the
// probes write (almost) nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 c_bf16x8 __attribute__((ext_vector_type(8)));
typedef float c_f32x16 __attribute__((ext_vector_type(16)));
typedef int c_i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t c_u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 4;

__global__ __launch_bounds__(kThreads) void mfma_bf16_loop(int iters, float* sink) {
  const int t = threadIdx.x;
  c_bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.001f * float((t + i) & 15));
    b[i] = (__bf16)(0.5f - 0.001f * float((t * 3 + i) & 15));
  }
  c_f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == -1.2345e-30f) sink[blockIdx.x * kThreads + t] = s;
}

__global__ __launch_bounds__(kThreads) void mfma_fp8_loop(int iters, float* sink) {
  const int t = threadIdx.x;
  c_i32x8 a, b;
  for (int i = 0; i < 8; ++i) {  // E4M3 bytes of moderate normal values
    a[i] = int(0x38383838u + uint32_t((t + i) & 3));
    b[i] = int(0x30303030u + uint32_t((t * 5 + i) & 3));
  }
  c_f32x16 acc[kChains];
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.0f;
  for (int c = 0; c < kChains; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == -1.2345e-30f) sink[blockIdx.x * kThreads + t] = s;
}

// Block b reads bytes [b * chunk, (b + 1) * chunk); chunk is a multiple of
// 16 * kThreads * kUnroll, so every 16-byte load of the block lies inside its
// chunk.  Each thread keeps kUnroll loads in flight.
constexpr int kUnroll = 8;
__global__ __launch_bounds__(kThreads) void stream_read(const c_u32x4* src, long long chunk16, uint32_t* sink) {
  const c_u32x4* p = src + (long long)blockIdx.x * chunk16 + threadIdx.x;
  c_u32x4 x = {0u, 0u, 0u, 0u};
  for (long long i = 0; i < chunk16; i += kThreads * kUnroll) {
    c_u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u];
  }
  const uint32_t v = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (v == 0x9e3779b9u) sink[blockIdx.x * kThreads + threadIdx.x] = v;
}

}  // namespace

extern "C" {

// flop of one launch: blocks * 4 wavefronts * iters * 4 chains * 32*32*16*2.
// sink: device, blocks * 256 floats (written only in the impossible case).
// 0 on success, else the hipError_t of the launch.
int moe_calib_mfma_bf16(int blocks, int iters, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || sink == nullptr) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_bf16_loop, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return int(hipGetLastError());
}

// flop of one launch: blocks * 4 wavefronts * iters * 4 chains * 32*32*64*2.
int moe_calib_mfma_fp8(int blocks, int iters, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || sink == nullptr) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_fp8_loop, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return int(hipGetLastError());
}

// Reads blocks * chunk bytes of src, chunk = floor(bytes / blocks) rounded
// down to a multiple of 32768; returns that byte count in *read (host).
// src 16-byte aligned; sink: device, blocks * 256 uint32.
int moe_calib_stream_read(const void* src, long long bytes, int blocks, uint32_t* sink, long long* read,
                          void* stream) {
  if (src == nullptr || sink == nullptr || read == nullptr || blocks <= 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return int(hipErrorInvalidValue);
  const long long unit = 16LL * kThreads * kUnroll;
  const long long chunk = bytes / blocks / unit * unit;
  if (chunk <= 0) return int(hipErrorInvalidValue);
  *read = chunk * blocks;
  hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const c_u32x4*>(src), chunk / 16, sink);
  return int(hipGetLastError());
}

}  // extern "C"
