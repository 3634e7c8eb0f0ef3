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
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

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

// split_bf16 of two values with the hardware conversion (round to nearest
// even, the same values): packed hi pair and packed lo pair.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const f32x2 f = {x0, x1};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  const f32x2 r = {x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
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

// cos/sin of (p0 + i) * theta_j into cs[i * h + j] for i < n, j < h.  Block-
// wide (every thread of the block calls it); the caller waits on a barrier
// before reading cs.  The angles at the coarse positions p0 + 8a and at the
// offsets b < 8 are evaluated as rope_cs does, and each entry is their
// product (angle addition in f32, about 2 ulp beyond rope_cs): a quarter of
// the evaluations of one rope_cs per entry.  scratch holds
// (ceil(n / 8) + 8) * h float2 and is free for the call.
__device__ __forceinline__ void rope_table(const RopeFreqs& r, int64_t p0, int n, int h, float2* cs,
                                           float2* scratch) {
  const int na = (n + 7) >> 3;
  for (int i = threadIdx.x; i < (na + 8) * h; i += blockDim.x) {
    const int a = i / h, j = i - a * h;
    const int64_t pos = a < na ? p0 + 8 * a : a - na;
    float c, s;
    rope_cs(static_cast<double>(pos), rope_freq(r, j), c, s);
    scratch[i] = make_float2(c, s);
  }
  __syncthreads();
  const float2* fine = scratch + na * h;
  for (int i = threadIdx.x; i < n * h; i += blockDim.x) {
    const int q = i / h, j = i - q * h;
    const float2 x = scratch[(q >> 3) * h + j], y = fine[(q & 7) * h + j];
    cs[i] = make_float2(x.x * y.x - x.y * y.y, x.x * y.y + x.y * y.x);
  }
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

// Inverse of order_key.
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// -0 -> +0, so that equal values get equal order keys.
__device__ __forceinline__ float plus_zero(float f) { return f == 0.f ? 0.f : f; }

// Cross-lane reductions without the LDS crossbar.  row16_max: the max over
// the 16 lanes of each DPP row (lanes 16r .. 16r + 15), in every lane of
// the row (rotations by 8, 4, 2, 1 within the row).  xor16_* / xor32_*:
// each lane combined with lane ^ 16 / lane ^ 32 (gfx950's permlane swaps;
// with both operands the same register, the two results hold the two
// partners, so their max or sum is the pair's in every lane).
template <int N>
__device__ __forceinline__ float dpp_row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_row_ror<8>(v));
  v = fmaxf(v, dpp_row_ror<4>(v));
  v = fmaxf(v, dpp_row_ror<2>(v));
  return fmaxf(v, dpp_row_ror<1>(v));
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
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

// Stage tiles filled by direct global -> LDS loads are unpadded rows of
// 2*D bytes whose 16-byte chunks are XOR-swizzled: chunk c of row r sits at
// position c ^ rswz<D>(r), which spreads both a 16-row operand read (one
// chunk per lane) and the fill over all banks.
template <int D>
__device__ __forceinline__ int rswz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

// Direct global -> LDS loads of 16 or 4 bytes per lane: lane l's bytes land
// at lds_wave + 16*l (4*l); lds_wave is the same in every lane of the wave.
// The host pass only needs the declaration.
__device__ __forceinline__ void load_lds16(const void* g, char* lds_wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds_wave, 16, 0, 0);
#endif
}
__device__ __forceinline__ void load_lds4(const void* g, char* lds_wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds_wave, 4, 0, 0);
#endif
}

// Waits until at most K vector-memory operations of this wave are
// outstanding and for its LDS operations, then meets the workgroup at a
// barrier.  Unlike __syncthreads, whose fence waits for every load in
// flight (direct LDS loads included), the loads of a later stage may stay
// in flight.  The empty asm statements keep the compiler from moving memory
// accesses across.
template <int K>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(K >= 0 && K < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((K & 15) | ((K >> 4) << 14) | (7 << 4));  // vmcnt(K) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Transposing LDS read of 16-bit elements (ds_read_b64_tr_b16): in each
// group of 16 lanes, lane j passes the address of 4 consecutive elements
// (8 bytes) of row j/4 at columns 4*(j%4) .. +3 of a 4 x 16 block, and lane
// i receives column i of the block's 4 rows (row 0 in the low half of .x).
__device__ __forceinline__ uint2 lds_read_tr16(const char* lds_addr) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
#if defined(__HIP_DEVICE_COMPILE__)
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds_addr));
#else
  const v4s v = {0, 0, 0, 0};
  (void)lds_addr;
#endif
  return make_uint2(static_cast<uint16_t>(v[0]) | (static_cast<uint32_t>(static_cast<uint16_t>(v[1])) << 16),
                    static_cast<uint16_t>(v[2]) | (static_cast<uint32_t>(static_cast<uint16_t>(v[3])) << 16));
}

}  // namespace hga
