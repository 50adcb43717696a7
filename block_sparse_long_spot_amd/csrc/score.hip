// Selector block scoring (SpotAttention §2.1 score formula, §2.3 per-block maximum).
//
// s[b][blk] = max_j sum_h w[b][h] * ReLU(q[b][h] . k[b][blk][j][h])
//
// HBM-bound: every selector key is read once. A key row (all heads of one key) is
// split into 16-byte chunks, one per lane, so a wave reads whole rows with
// contiguous 16-byte loads: 8 elements per lane for fp32/bf16 keys (fp32 takes two
// loads), 16 for the 8-bit formats, 32 for the 4-bit ones (exactly one scale group).
// Lanes of one head reduce their partial dots with cross-lane adds (DPP inside a row
// of 16 lanes), apply ReLU and the head weight, then lanes of one row add the heads.
//
// Quantised keys (§5.3, Appendix G) are decoded in registers: FP8 E4M3 and FP4 E2M1
// by the gfx950 conversion instructions (two elements per instruction), INT8 by a
// byte-to-float conversion of the code biased by +128 (the bias is removed once per
// dot through the sum of the query slice), INT4 by nibble sign extension. Scales are
// factored out of the dot: one multiply per 16-byte chunk (group formats) or per dot
// (per-tensor formats). The query, read once per thread, may use any format.
#include "device_common.h"
#include "spot_internal.h"

namespace spot {
namespace {

// elements of d_idx in one lane's 16-byte chunk of a key row
template <int KF>
constexpr int key_chunk() {
  return (KF == kInt4 || KF == kFp4) ? 32 : ((KF == kInt8 || KF == kFp8) ? 16 : 8);
}

// E8M0 scale byte: 2^(x - 127) (x = 0 is the subnormal 2^-127)
__device__ __forceinline__ float e8m0_to_f(uint32_t x) {
  return __uint_as_float(x ? (x << 23) : 0x00400000u);
}

// Element e (flat index) of a selector tensor in format fmt with its scale array. Used
// for the query only, once per thread, so a run-time switch is fine.
__device__ float selector_elem(const void* p, int fmt, const void* sc, size_t e) {
  switch (fmt) {
    case kF32:
      return static_cast<const float*>(p)[e];
    case kBF16:
      return bf16_to_f(static_cast<const uint16_t*>(p)[e]);
    case kInt8:
      return static_cast<float>(static_cast<const int8_t*>(p)[e]) *
             *static_cast<const float*>(sc);
    case kFp8: {
      const uint32_t byte = static_cast<const uint8_t*>(p)[e];
      return __builtin_amdgcn_cvt_pk_f32_fp8(byte, false)[0] * *static_cast<const float*>(sc);
    }
    case kInt4: {
      const uint32_t byte = static_cast<const uint8_t*>(p)[e >> 1];
      const int code = static_cast<int>(byte << (28 - 4 * (e & 1))) >> 28;
      return static_cast<float>(code) *
             half_bits_to_f(static_cast<const uint16_t*>(sc)[e >> 5]);
    }
    default: {  // kFp4
      const uint32_t byte = static_cast<const uint8_t*>(p)[e >> 1];
      const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);
      return ((e & 1) ? v[1] : v[0]) * e8m0_to_f(static_cast<const uint8_t*>(sc)[e >> 5]);
    }
  }
}

// sum of q[8j .. 8j+7] * fp4 elements of byte lane J of word w (the two nibbles of
// each byte, low first)
template <int J>
__device__ __forceinline__ float fp4_dot2(uint32_t w, const float* q, float a) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, J);
  a = fmaf(q[2 * J], v[0], a);
  return fmaf(q[2 * J + 1], v[1], a);
}

// QF: kF32 or kBF16 (vector loads of the query) or -1 (any format, element by element).
// R > 1 (one key per block only): each wave scores R consecutive groups of blocks, all
// their key loads issued before any is used, so a launch needs R times fewer
// work-groups for the same bytes in flight.
template <int QF, int KF, int DIDX, int R>
__global__ __launch_bounds__(256) void select_score_kernel(
    const void* __restrict__ sel_q, int q_fmt, const void* __restrict__ sel_q_scale,
    const float* __restrict__ sel_w, const void* __restrict__ sel_k,
    const void* __restrict__ sel_k_scale, float* __restrict__ scores, int nb, int kpb, int H,
    int lpr_log2) {
  constexpr int CH = key_chunk<KF>();   // elements per lane per key row
  constexpr int LPH = DIDX / CH;        // lanes per selector head
  const int LPR = 1 << lpr_log2;        // lanes per key row = H * LPH
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gl = lane & (LPR - 1);
  const int head = gl / LPH;
  const int part = gl % LPH;
  const int per_wave = 64 >> lpr_log2;
  const int b = blockIdx.y;
  // first block of this lane group; round r adds r * per_wave
  const int blk = ((blockIdx.x * 4 + wave) * R) * per_wave + (lane >> lpr_log2);
  const bool valid = blk < nb;
  const int blk_c = valid ? blk : nb - 1;  // lanes past the end read a valid row

  float qv[CH];
  const size_t q0 = ((size_t)b * H + head) * DIDX + part * CH;
  if constexpr (QF == kF32 || QF == kBF16) {
    typedef typename std::conditional<QF == kF32, float, uint16_t>::type QT;
    const QT* qp = static_cast<const QT*>(sel_q) + q0;
#pragma unroll
    for (int c = 0; c < CH; c += 8) load8(qp + c, qv + c);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) qv[c] = selector_elem(sel_q, q_fmt, sel_q_scale, q0 + c);
  }
  const float wh = sel_w[(size_t)b * H + head];
  float kscale = 1.f, qsum = 0.f;
  if constexpr (KF == kInt8 || KF == kFp8) kscale = *static_cast<const float*>(sel_k_scale);
  if constexpr (KF == kInt8) {
#pragma unroll
    for (int c = 0; c < CH; ++c) qsum += qv[c];
  }

  // score of selector key j of this lane group's block (all lanes of the group return it)
  auto key_score = [&](const u32x4_t& raw, const u32x4_t& raw2, uint32_t sh) {
    float dot = 0.f;
    if constexpr (KF == kInt4) {
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          // nibble n of word k is element 8k+n; shift it to the top, sign-extend down
          const int code = static_cast<int>(raw[k] << (28 - 4 * n)) >> 28;
          a = fmaf(qv[k * 8 + n], static_cast<float>(code), a);
        }
      }
      dot = a * half_bits_to_f(static_cast<uint16_t>(sh));
    } else if constexpr (KF == kFp4) {
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a = fp4_dot2<0>(raw[k], qv + 8 * k, a);
        a = fp4_dot2<1>(raw[k], qv + 8 * k, a);
        a = fp4_dot2<2>(raw[k], qv + 8 * k, a);
        a = fp4_dot2<3>(raw[k], qv + 8 * k, a);
      }
      dot = a * e8m0_to_f(sh);
    } else if constexpr (KF == kInt8) {
      // byte + 128 (the sign bit flipped) is the code plus 128, converted directly
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t u = raw[k] ^ 0x80808080u;
#pragma unroll
        for (int n = 0; n < 4; ++n)
          a = fmaf(qv[4 * k + n], static_cast<float>((u >> (8 * n)) & 0xffu), a);
      }
      dot = (a - 128.f * qsum) * kscale;
    } else if constexpr (KF == kFp8) {
      float a = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(raw[k], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(raw[k], true);
        a = fmaf(qv[4 * k], lo[0], a);
        a = fmaf(qv[4 * k + 1], lo[1], a);
        a = fmaf(qv[4 * k + 2], hi[0], a);
        a = fmaf(qv[4 * k + 3], hi[1], a);
      }
      dot = a * kscale;
    } else if constexpr (KF == kF32) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        dot = fmaf(qv[n], __uint_as_float(raw[n]), dot);
        dot = fmaf(qv[4 + n], __uint_as_float(raw2[n]), dot);
      }
    } else {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        dot = fmaf(qv[2 * n], bf16_lo(raw[n]), dot);
        dot = fmaf(qv[2 * n + 1], bf16_hi(raw[n]), dot);
      }
    }
    dot = group_sum_dpp<LPH>(dot);
    // every lane of a head now holds that head's term; add the heads of the row
    return group_sum_dpp_rt<LPH>(wh * fmaxf(dot, 0.f), lpr_log2);
  };
  // this lane's 16-byte chunk (two for fp32 keys) of key j of block bc, and its group scale
  auto load_key_of = [&](int bc, int j, u32x4_t& raw, u32x4_t& raw2, uint32_t& sh) {
    const size_t row = ((size_t)b * nb + bc) * kpb + j;
    if constexpr (KF == kInt4 || KF == kFp4) {
      const uint8_t* cp = static_cast<const uint8_t*>(sel_k) + (row * H + head) * (DIDX / 2) +
                          part * 16;
      raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cp));
      const size_t si = (row * H + head) * (DIDX / 32) + part;
      if constexpr (KF == kInt4)
        sh = static_cast<const uint16_t*>(sel_k_scale)[si];
      else
        sh = static_cast<const uint8_t*>(sel_k_scale)[si];
    } else if constexpr (KF == kInt8 || KF == kFp8) {
      const uint8_t* cp = static_cast<const uint8_t*>(sel_k) + (row * H + head) * DIDX +
                          part * 16;
      raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cp));
    } else {
      typedef typename std::conditional<KF == kF32, float, uint16_t>::type KT;
      const KT* kp = static_cast<const KT*>(sel_k) + (row * H + head) * DIDX + part * CH;
      raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp));
      if constexpr (KF == kF32)
        raw2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + 4));
    }
  };

  auto load_key = [&](int j, u32x4_t& raw, u32x4_t& raw2, uint32_t& sh) {
    load_key_of(blk_c, j, raw, raw2, sh);
  };
  if constexpr (R > 1) {
    // one key per block: R groups of blocks, loads first
    u32x4_t r[R], r2[R];
    uint32_t sc[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int bu = blk + u * per_wave;
      load_key_of(bu < nb ? bu : nb - 1, 0, r[u], r2[u], sc[u]);
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int bu = blk + u * per_wave;
      const float v = key_score(r[u], r2[u], sc[u]);
      if (bu < nb && gl == 0) scores[(size_t)b * nb + bu] = v;
    }
    return;
  }
  // Keys of a block are read KU at a time so their loads overlap (per-token keys): 8
  // (16 for the 4-bit formats, whose key rows are shortest) keep enough bytes in flight
  // per wave (measured at 16 bf16 keys of 4 x 128 per block: 8 at a time 5 % faster
  // than 4, 16 no faster).
  constexpr int KU = CH == 32 ? 16 : 8;
  float best = -INFINITY;
  int j = 0;
  for (; j + KU <= kpb; j += KU) {
    u32x4_t r[KU], r2[KU];
    uint32_t sc[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) load_key(j + u, r[u], r2[u], sc[u]);
#pragma unroll
    for (int u = 0; u < KU; ++u) best = fmaxf(best, key_score(r[u], r2[u], sc[u]));
  }
  for (; j + 4 <= kpb; j += 4) {
    u32x4_t r[4], r2[4];
    uint32_t sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) load_key(j + u, r[u], r2[u], sc[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) best = fmaxf(best, key_score(r[u], r2[u], sc[u]));
  }
  for (; j < kpb; ++j) {
    u32x4_t r, r2;
    uint32_t sc;
    load_key(j, r, r2, sc);
    best = fmaxf(best, key_score(r, r2, sc));
  }
  if (valid && gl == 0) scores[(size_t)b * nb + blk] = best;
}

template <int QF, int KF>
hipError_t launch_kf(const void* sel_q, int q_fmt, const void* sel_q_scale, const float* sel_w,
                     const void* sel_k, const void* sel_k_scale, float* scores, int B, int nb,
                     int kpb, int H, int d_idx, hipStream_t stream) {
  const int lpr = H * (d_idx / key_chunk<KF>());
  int lpr_log2 = 0;
  while ((1 << lpr_log2) < lpr) ++lpr_log2;
  const int per_wg = 4 * (64 >> lpr_log2);
  // One key per block: R rounds per wave, the largest of 1, 2 and 4 that still leaves
  // at least 1024 work-groups (measured at 128K: batch 8 takes 2.3 us with 1024
  // work-groups of 2 rounds, 2.5 with 512 of 4 or 2048 of 1; batch 1, 256 work-groups
  // of 1 round, 1.9 us, 128 of 2 2.0)
  const long wg1 = ((long)nb + per_wg - 1) / per_wg * B;
  const int R = kpb != 1 ? 1 : (wg1 >= 4096 ? 4 : (wg1 >= 2048 ? 2 : 1));
  dim3 grid((unsigned)(((long)nb + per_wg * R - 1) / (per_wg * R)), B), block(256);
#define SPOT_SCORE(DIDX, RR)                                                                 \
  hipLaunchKernelGGL((select_score_kernel<QF, KF, DIDX, RR>), grid, block, 0, stream, sel_q,   \
                     q_fmt, sel_q_scale, sel_w, sel_k, sel_k_scale, scores, nb, kpb, H,       \
                     lpr_log2)
#define SPOT_SCORE_R(DIDX) \
  if (R == 4)              \
    SPOT_SCORE(DIDX, 4);   \
  else if (R == 2)         \
    SPOT_SCORE(DIDX, 2);   \
  else                     \
    SPOT_SCORE(DIDX, 1);
  switch (d_idx) {
    case 32: SPOT_SCORE_R(32); break;
    case 64: SPOT_SCORE_R(64); break;
    default: SPOT_SCORE_R(128); break;
  }
#undef SPOT_SCORE_R
#undef SPOT_SCORE
  return hipGetLastError();
}

template <int QF>
hipError_t launch_q(const void* sel_q, int q_fmt, const void* sel_q_scale, const float* sel_w,
                    const void* sel_k, const void* sel_k_scale, int k_fmt, float* scores, int B,
                    int nb, int kpb, int H, int d_idx, hipStream_t stream) {
#define SPOT_KF(KF)                                                                         \
  return launch_kf<QF, KF>(sel_q, q_fmt, sel_q_scale, sel_w, sel_k, sel_k_scale, scores, B, \
                           nb, kpb, H, d_idx, stream)
  switch (k_fmt) {
    case kF32: SPOT_KF(kF32);
    case kBF16: SPOT_KF(kBF16);
    case kInt8: SPOT_KF(kInt8);
    case kFp8: SPOT_KF(kFp8);
    case kInt4: SPOT_KF(kInt4);
    default: SPOT_KF(kFp4);
  }
#undef SPOT_KF
}

}  // namespace

hipError_t launch_select_score(const void* sel_q, int q_fmt, const void* sel_q_scale,
                               const float* sel_w, const void* sel_k, const void* sel_k_scale,
                               int k_fmt, float* scores, int B, int nb, int kpb, int H,
                               int d_idx, hipStream_t stream) {
  if (q_fmt == kF32)
    return launch_q<kF32>(sel_q, q_fmt, sel_q_scale, sel_w, sel_k, sel_k_scale, k_fmt, scores,
                          B, nb, kpb, H, d_idx, stream);
  if (q_fmt == kBF16)
    return launch_q<kBF16>(sel_q, q_fmt, sel_q_scale, sel_w, sel_k, sel_k_scale, k_fmt, scores,
                           B, nb, kpb, H, d_idx, stream);
  return launch_q<-1>(sel_q, q_fmt, sel_q_scale, sel_w, sel_k, sel_k_scale, k_fmt, scores, B,
                      nb, kpb, H, d_idx, stream);
}

}  // namespace spot
