// Quantisation of selector keys into the cache formats (SpotAttention §5.3 and
// Appendix G: the selector is trained in BF16 and its key cache quantised at
// inference) - the write side used when a new token's key is appended.
//
// One thread per group of 32 consecutive elements of a row: it reads the group (two
// or four 16-byte loads), chooses the group scale where the format has one, encodes
// the codes and writes them with 16-byte stores. Where a float decides an integer
// code the decision is a correctly rounded float32 quotient rounded to nearest even
// (rintf); the FP4 exponent and the E4M3 encoding are exact integer arithmetic on
// the binary exponent. Memory-bound and tiny at decode (one key row per sequence).
#include "device_common.h"
#include "spot_internal.h"

namespace spot {
namespace {

// E4M3 code of y with |y| <= 448 (saturated by the caller): the codes of the finite
// magnitudes are increasing, so the nearest one is an integer rounding of |y| on the
// grid of its binade (ties to even), and a carry out of the mantissa steps into the
// next exponent by itself. Sign bit from y (a negative value rounding to 0 is -0).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const float a = fabsf(y);
  uint32_t mag;
  if (a < 0x1p-6f) {
    mag = static_cast<uint32_t>(rintf(a * 512.f));          // subnormals: steps of 2^-9
  } else {
    int k;
    frexpf(a, &k);                                          // a = m * 2^k, m in [0.5, 1)
    const int E = k - 1;                                    // a in [2^E, 2^(E+1))
    mag = static_cast<uint32_t>(E * 8 + 48) +
          static_cast<uint32_t>(rintf(ldexpf(a, 3 - E)));   // (E + 7) * 8 + mantissa
  }
  return mag | (signbit(y) ? 0x80u : 0u);
}

// E2M1 magnitude code of |y| <= 6: nearest value, ties to the even code
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  uint32_t c = 0;
  c += a > 0.25f;   // 0 | 0.5   (tie -> 0)
  c += a >= 0.75f;  // 0.5 | 1   (tie -> 1)
  c += a > 1.25f;   // 1 | 1.5   (tie -> 1)
  c += a >= 1.75f;  // 1.5 | 2   (tie -> 2)
  c += a > 2.5f;    // 2 | 3     (tie -> 2)
  c += a >= 3.5f;   // 3 | 4     (tie -> 4)
  c += a > 5.f;     // 4 | 6     (tie -> 4)
  return c | (signbit(y) ? 8u : 0u);
}

template <typename ST, int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(const ST* __restrict__ src,
                                                       uint8_t* __restrict__ codes,
                                                       void* __restrict__ scales,
                                                       const float* __restrict__ tscale,
                                                       long n_groups) {
  const long gi = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= n_groups) return;
  float x[32];
#pragma unroll
  for (int c = 0; c < 32; c += 8) load8(src + gi * 32 + c, x + c);
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(x[c]));
  u32x4_t out[2];
  if constexpr (FMT == kInt4) {
    const _Float16 s16 = static_cast<_Float16>(amax / 7.f);
    const float s = static_cast<float>(s16);
    static_cast<_Float16*>(scales)[gi] = s16;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const float q = s > 0.f ? fminf(fmaxf(rintf(x[8 * w + n] / s), -8.f), 7.f) : 0.f;
        word |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xFu) << (4 * n);
      }
      out[0][w] = word;
    }
  } else if constexpr (FMT == kFp4) {
    int e = -127;
    if (amax > 0.f) {
      int k;
      const float m = frexpf(amax, &k);
      e = m <= 0.75f ? k - 3 : k - 2;   // smallest e with amax <= 6 * 2^e
      e = min(max(e, -127), 127);
    }
    static_cast<uint8_t*>(scales)[gi] = static_cast<uint8_t>(e + 127);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) word |= e2m1_code(ldexpf(x[8 * w + n], -e)) << (4 * n);
      out[0][w] = word;
    }
  } else if constexpr (FMT == kInt8) {
    const float s = *tscale;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const float q = fminf(fmaxf(rintf(x[4 * w + n] / s), -127.f), 127.f);
        word |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xFFu) << (8 * n);
      }
      out[w / 4][w % 4] = word;
    }
  } else {  // kFp8
    const float s = *tscale;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 4; ++n)
        word |= e4m3_code(fminf(fmaxf(x[4 * w + n] / s, -448.f), 448.f)) << (8 * n);
      out[w / 4][w % 4] = word;
    }
  }
  constexpr int BYTES = (FMT == kInt4 || FMT == kFp4) ? 16 : 32;
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + gi * BYTES);
  dst[0] = out[0];
  if constexpr (BYTES == 32) dst[1] = out[1];
}

template <typename ST>
hipError_t launch_st(const void* src, int fmt, void* codes, void* scales,
                     const float* tensor_scale, long n_groups, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n_groups + 255) / 256)), block(256);
  const ST* s = static_cast<const ST*>(src);
  uint8_t* c = static_cast<uint8_t*>(codes);
  switch (fmt) {
    case kInt4:
      hipLaunchKernelGGL((quantize_kernel<ST, kInt4>), grid, block, 0, stream, s, c, scales,
                         tensor_scale, n_groups);
      break;
    case kFp4:
      hipLaunchKernelGGL((quantize_kernel<ST, kFp4>), grid, block, 0, stream, s, c, scales,
                         tensor_scale, n_groups);
      break;
    case kInt8:
      hipLaunchKernelGGL((quantize_kernel<ST, kInt8>), grid, block, 0, stream, s, c, scales,
                         tensor_scale, n_groups);
      break;
    default:
      hipLaunchKernelGGL((quantize_kernel<ST, kFp8>), grid, block, 0, stream, s, c, scales,
                         tensor_scale, n_groups);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_selector(const void* src, bool src_bf16, int fmt, void* codes,
                                    void* scales, const float* tensor_scale, long n_groups,
                                    hipStream_t stream) {
  if (src_bf16)
    return launch_st<uint16_t>(src, fmt, codes, scales, tensor_scale, n_groups, stream);
  return launch_st<float>(src, fmt, codes, scales, tensor_scale, n_groups, stream);
}

}  // namespace spot
