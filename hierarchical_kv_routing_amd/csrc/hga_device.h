// Device-side helpers shared by the gfx950 kernels: element loads, bf16
// rounding, RoPE angles, matrix-core wrappers and order-preserving keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hga_internal.h"

namespace hga {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

union Pack8 {
  bf16x8 v;
  uint4 q;
  uint32_t u[4];
  uint16_t h[8];
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bf16 pair (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Split x into hi + lo with hi = bf16(x), lo = bf16(x - hi): hi*y + lo*y
// recovers x*y to about 2^-17 relative.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// Eight consecutive elements as f32 (16-byte aligned source).
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float out[8]) {
  if constexpr (BF16) {
    uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(u[i] << 16);
      out[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, int64_t elem) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[elem]);
  else return static_cast<const float*>(base)[elem];
}

template <bool BF16>
__device__ __forceinline__ void store1(void* base, int64_t elem, float x) {
  if constexpr (BF16) static_cast<uint16_t*>(base)[elem] = f32_to_bf16(x);
  else static_cast<float*>(base)[elem] = x;
}

// cos/sin of pos * freq: the angle is formed and reduced to [-pi, pi] in
// double (two-part 2*pi), then evaluated in f32.
__device__ __forceinline__ void rope_cs(double pos, double freq, float& c, float& s) {
  const double kTwoPiHi = 6.283185307179586;
  const double kTwoPiLo = 2.4492935982947064e-16;
  const double kInvTwoPi = 0.15915494309189535;
  double a = pos * freq;
  double k = rint(a * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, a);
  r = fma(-k, kTwoPiLo, r);
  sincosf(static_cast<float>(r), &s, &c);
}

// theta_i as the product of the factors of the set bits of i (fixed order,
// so every kernel forms the same value).
__device__ __forceinline__ double rope_freq(const RopeFreqs& r, int i) {
  double f = 1.0;
#pragma unroll
  for (int b = 0; b < 6; ++b) f = ((i >> b) & 1) ? f * r.step[b] : f;
  return f;
}

// Rotation position of the token at absolute position p: p mod period when
// positions wrap.  Periods are multiples of C, so a caller wraps the first
// position of a chunk or group once and adds in-block offsets to it.
__device__ __forceinline__ int64_t rope_base(const RopeFreqs& r, int64_t p) {
  return r.period > 0 ? p % r.period : p;
}

// Larger float -> larger unsigned key (total order on finite values).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Matrix-core wrappers (gfx950 double-rate bf16 forms).
//   16x16x32: A[m][k] m = lane%16; B[k][n] n = lane%16; each lane brings 8
//             k-values (the same k slots for A and B);
//             D[m][n]: n = lane%16, m = 4*(lane/16) + j, j < 4.
//   32x32x16: A m = lane%32, B n = lane%32, 8 k-values per lane;
//             D[m][n]: n = lane%32, m = 8*(j/4) + 4*(lane/32) + (j%4), j < 16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace hga
