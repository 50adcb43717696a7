// Device helpers shared by the libspot kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spot {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// bfloat16 is the upper half of a binary32: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// IEEE binary16 bits to fp32 (exact).
__device__ __forceinline__ float half_bits_to_f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Eight consecutive elements widened to fp32. `p` is 16-byte aligned for bf16 and
// 32-byte aligned for fp32.
__device__ __forceinline__ void load8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  o[0] = bf16_lo(a.x); o[1] = bf16_hi(a.x);
  o[2] = bf16_lo(a.y); o[3] = bf16_hi(a.y);
  o[4] = bf16_lo(a.z); o[5] = bf16_hi(a.z);
  o[6] = bf16_lo(a.w); o[7] = bf16_hi(a.w);
}

// The same for data read exactly once (non-temporal loads).
__device__ __forceinline__ void load8_stream(const float* p, float* o) {
  const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  const u32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = __uint_as_float(a[i]);
    o[4 + i] = __uint_as_float(b[i]);
  }
}
__device__ __forceinline__ void load8_stream(const uint16_t* p, float* o) {
  const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = bf16_lo(a[i]);
    o[2 * i + 1] = bf16_hi(a[i]);
  }
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < WIDTH; o <<= 1) v += shfl_xor_f(v, o);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < WIDTH; o <<= 1) v = fmaxf(v, shfl_xor_f(v, o));
  return v;
}

// Order-preserving map of a binary32 onto uint32 (larger float -> larger key).
// -0.0 must be folded onto +0.0 by the caller.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace spot
