// Peak microbenchmarks for the roofline denominators, measured on the device
// the path runs on (vendor figures are the other denominator).
//
//  * hga_peak_mfma: back-to-back v_mfma_f32_32x32x16_bf16 on register
//    operands, 4 independent accumulators per wave, many waves per SIMD:
//    the dense bf16 matrix rate the attention kernel's products can reach.
//  * hga_peak_stream: a streaming copy (16-byte loads and stores, grid-stride)
//    of a caller buffer: the HBM rate a bandwidth-bound kernel can reach.
//
// Both are measurement tools beside the library (libhga_peak.so); nothing on
// the routed-attention path calls them.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__global__ __launch_bounds__(256) void mfma_loop(float* sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1.0f + 1e-3f * static_cast<float>((threadIdx.x + i) & 7));
    b[i] = static_cast<__bf16>(1.0f - 1e-3f * static_cast<float>((threadIdx.x * 3 + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void stream_copy(const uint4* src, uint4* dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

}  // namespace

extern "C" {

// Launches `blocks` workgroups of 256 threads, each wave issuing 4*iters
// 32x32x16 bf16 MFMAs (32768 flops each).  sink: device buffer of
// blocks*256 floats.  Returns the HIP error code; flops = blocks*4*4*iters*32768.
int hga_peak_mfma(float* sink, int blocks, int iters, void* stream) {
  if (sink == nullptr || blocks <= 0 || iters <= 0) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), sink,
                     iters);
  return static_cast<int>(hipGetLastError());
}

// Copies `bytes` (a multiple of 16, 16-byte aligned buffers) from src to dst.
int hga_peak_stream(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0)
    return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(stream_copy, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
