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

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// An LDS address of a kernel's shared arrays as the LDS-space pointer that the
// transposing LDS read takes.
__device__ __forceinline__ lds_s16x4_t* lds_s16x4(const uint16_t* p) {
  return (lds_s16x4_t*)((__attribute__((address_space(3))) uint16_t*)p);
}

// B operand (k = 8 tokens, n = 16 dims) of v_mfma_f32_16x16x32_bf16 from a row-major
// [token][dim] bf16 tile in LDS, through gfx950's transposing LDS read
// (ds_read_b64_tr_b16). In each 16-lane group, source lane `row` passes the address of
// tile row r0 + row/4, column c0 + 4(row%4); lane `row` then receives column c0 + row
// of rows r0 .. r0+3 (k = 0..3) and of rows r0+16 .. r0+19 (k = 4..7). `stride` is the
// tile's row stride in elements.
__device__ __forceinline__ bf16x8_t lds_tr_b_operand(const uint16_t* p, int stride) {
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_s16x4(p));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_s16x4(p + 16 * stride));
  const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  const u32x4_t v = {l2[0], l2[1], h2[0], h2[1]};
  return __builtin_bit_cast(bf16x8_t, v);
}

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

// ---- wave64 scans on the DPP network (gfx9 row_shr / row_bcast controls): each step
// reads a neighbouring lane's register inside the VALU instruction, no LDS traffic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ unsigned long long dpp_or_zero(unsigned long long v) {
  const uint32_t lo = dpp_or_zero<CTRL, ROW_MASK>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_or_zero<CTRL, ROW_MASK>(static_cast<uint32_t>(v >> 32));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
// Inclusive prefix sum over the 64 lanes (lane i gets the sum of lanes 0..i).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T x) {
  x += dpp_or_zero<0x111, 0xf>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xf>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xf>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xf>(x);  // row_shr:8   (now a scan inside each row of 16)
  x += dpp_or_zero<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_or_zero<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float x) {
  // lanes without a valid source (or outside ROW_MASK) see their own value
  const int xi = __float_as_int(x);
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, CTRL, ROW_MASK, 0xf, false)));
}
// Maximum over the 64 lanes, valid in lane 63 (a running maximum in lane order).
__device__ __forceinline__ float wave_max_to_last(float x) {
  x = dpp_max_step<0x111, 0xf>(x);
  x = dpp_max_step<0x112, 0xf>(x);
  x = dpp_max_step<0x114, 0xf>(x);
  x = dpp_max_step<0x118, 0xf>(x);
  x = dpp_max_step<0x142, 0xa>(x);
  x = dpp_max_step<0x143, 0xc>(x);
  return x;
}
template <typename T>
__device__ __forceinline__ T lane_value(T x, int lane) {
  if constexpr (sizeof(T) == 8) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), lane);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(x >> 32), lane);
    return static_cast<T>((static_cast<unsigned long long>(hi) << 32) | lo);
  } else {
    return static_cast<T>(__builtin_amdgcn_readlane(static_cast<int>(x), lane));
  }
}

// Value of another lane of the same row of 16 lanes, on the DPP network (CTRL is a DPP
// row control: quad_perm, row_ror, row mirror, ...).
template <int CTRL>
__device__ __forceinline__ float dpp_rot(float x) {
  const int xi = __float_as_int(x);
  return __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, CTRL, 0xf, 0xf, false));
}

// Reductions across the rows of 16 lanes with gfx950's lane-swap instructions (VALU,
// no LDS round trip). With both operands equal, v_permlane16_swap returns in every
// lane the values of lanes l & ~16 and l | 16, and v_permlane32_swap those of lanes
// l & 31 and (l & 31) + 32: their sum or maximum is the reduction over the lane pair
// l, l ^ 16 (resp. l, l ^ 32), computed in the same order in both lanes.
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over aligned groups of W lanes (W a power of two <= 64), result in every lane of
// the group, for values already summed over aligned groups of FROM lanes (every lane of
// such a group holds the same value; FROM = 1 for arbitrary values). Inside a row of 16
// the steps run on the DPP network (quad_perm swaps, then row half-mirror and mirror,
// which pair each lane with one in the other half of its group of 8 or 16); across rows
// they are lane swaps.
template <int W, int FROM = 1>
__device__ __forceinline__ float group_sum_dpp(float x) {
  if constexpr (FROM <= 1 && W >= 2) x += dpp_rot<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (FROM <= 2 && W >= 4) x += dpp_rot<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (FROM <= 4 && W >= 8) x += dpp_rot<0x141>(x);   // row_half_mirror
  if constexpr (FROM <= 8 && W >= 16) x += dpp_rot<0x140>(x);  // row_mirror
  if constexpr (FROM <= 16 && W >= 32) x = xor16_sum(x);
  if constexpr (FROM <= 32 && W >= 64) x = xor32_sum(x);
  return x;
}
// The same with the group size 2^log2w chosen at run time (uniform across the wave).
template <int FROM>
__device__ __forceinline__ float group_sum_dpp_rt(float x, int log2w) {
  switch (log2w) {
    case 0: return x;
    case 1: return group_sum_dpp<2, FROM>(x);
    case 2: return group_sum_dpp<4, FROM>(x);
    case 3: return group_sum_dpp<8, FROM>(x);
    case 4: return group_sum_dpp<16, FROM>(x);
    case 5: return group_sum_dpp<32, FROM>(x);
    default: return group_sum_dpp<64, FROM>(x);
  }
}

// Order-preserving map of a binary32 onto uint32 (larger float -> larger key).
// -0.0 must be folded onto +0.0 by the caller.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace spot
