// Selector block scoring (SpotAttention §2.1 score formula, §2.3 per-block maximum).
//
// s[b][blk] = max_j sum_h w[b][h] * ReLU(q[b][h] . k[b][blk][j][h])
//
// HBM-bound: every selector key is read once. A key row (all heads of one key) is
// split into 16-byte chunks, one per lane, so a wave reads whole rows with
// contiguous 16-byte loads: 8 elements per lane for fp32/bf16 keys (fp32 takes two
// loads), 32 INT4 codes per lane for the quantised cache (exactly one fp16 scale
// group). Lanes of one head reduce their partial dots with cross-lane adds (DPP inside
// a row of 16 lanes), apply ReLU and the head weight, then lanes of one row add the heads.
#include "device_common.h"
#include "spot_internal.h"

namespace spot {
namespace {

template <typename QT, int KK, int DIDX>
__global__ __launch_bounds__(256) void select_score_kernel(
    const QT* __restrict__ sel_q, const float* __restrict__ sel_w,
    const void* __restrict__ sel_k, const uint16_t* __restrict__ sel_scale,
    float* __restrict__ scores, int nb, int kpb, int H, int lpr_log2) {
  constexpr int CH = (KK == kKeyInt4) ? 32 : 8;  // elements per lane per key row
  constexpr int LPH = DIDX / CH;                 // lanes per selector head
  const int LPR = 1 << lpr_log2;                 // lanes per key row = H * LPH
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gl = lane & (LPR - 1);
  const int head = gl / LPH;
  const int part = gl % LPH;
  const int per_wave = 64 >> lpr_log2;
  const int b = blockIdx.y;
  const int blk = (blockIdx.x * 4 + wave) * per_wave + (lane >> lpr_log2);
  const bool valid = blk < nb;
  const int blk_c = valid ? blk : nb - 1;  // lanes past the end read a valid row

  float qv[CH];
  const QT* qp = sel_q + ((size_t)b * H + head) * DIDX + part * CH;
#pragma unroll
  for (int c = 0; c < CH; c += 8) load8(qp + c, qv + c);
  const float wh = sel_w[(size_t)b * H + head];

  // score of selector key j of this lane group's block (all lanes of the group return it)
  auto key_score = [&](int j, const u32x4_t& raw, const u32x4_t& raw2, uint16_t sh) {
    float dot = 0.f;
    if constexpr (KK == kKeyInt4) {
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
      dot = a * half_bits_to_f(sh);
    } else if constexpr (KK == kKeyF32) {
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
  // this lane's 16-byte chunk (two for fp32 keys) of key j
  auto load_key = [&](int j, u32x4_t& raw, u32x4_t& raw2, uint16_t& sh) {
    const size_t row = ((size_t)b * nb + blk_c) * kpb + j;
    if constexpr (KK == kKeyInt4) {
      const uint8_t* cp = static_cast<const uint8_t*>(sel_k) + (row * H + head) * (DIDX / 2) +
                          part * 16;
      raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cp));
      sh = sel_scale[(row * H + head) * (DIDX / 32) + part];
    } else {
      typedef typename std::conditional<KK == kKeyF32, float, uint16_t>::type KT;
      const KT* kp = static_cast<const KT*>(sel_k) + (row * H + head) * DIDX + part * CH;
      raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp));
      if constexpr (KK == kKeyF32)
        raw2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + 4));
    }
  };

  // keys of a block are read four at a time so their loads overlap (per-token keys)
  float best = -INFINITY;
  int j = 0;
  for (; j + 4 <= kpb; j += 4) {
    u32x4_t r[4], r2[4];
    uint16_t sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) load_key(j + u, r[u], r2[u], sc[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) best = fmaxf(best, key_score(j + u, r[u], r2[u], sc[u]));
  }
  for (; j < kpb; ++j) {
    u32x4_t r, r2;
    uint16_t sc;
    load_key(j, r, r2, sc);
    best = fmaxf(best, key_score(j, r, r2, sc));
  }
  if (valid && gl == 0) scores[(size_t)b * nb + blk] = best;
}

template <typename QT, int KK>
hipError_t launch_kk(const void* sel_q, const float* sel_w, const void* sel_k,
                     const void* sel_scale, float* scores, int B, int nb, int kpb, int H,
                     int d_idx, hipStream_t stream) {
  const int ch = (KK == kKeyInt4) ? 32 : 8;
  const int lpr = H * (d_idx / ch);
  int lpr_log2 = 0;
  while ((1 << lpr_log2) < lpr) ++lpr_log2;
  const int per_wg = 4 * (64 >> lpr_log2);
  dim3 grid((nb + per_wg - 1) / per_wg, B), block(256);
  const QT* q = static_cast<const QT*>(sel_q);
  const uint16_t* sc = static_cast<const uint16_t*>(sel_scale);
  switch (d_idx) {
    case 32:
      hipLaunchKernelGGL((select_score_kernel<QT, KK, 32>), grid, block, 0, stream, q, sel_w,
                         sel_k, sc, scores, nb, kpb, H, lpr_log2);
      break;
    case 64:
      hipLaunchKernelGGL((select_score_kernel<QT, KK, 64>), grid, block, 0, stream, q, sel_w,
                         sel_k, sc, scores, nb, kpb, H, lpr_log2);
      break;
    default:
      hipLaunchKernelGGL((select_score_kernel<QT, KK, 128>), grid, block, 0, stream, q, sel_w,
                         sel_k, sc, scores, nb, kpb, H, lpr_log2);
      break;
  }
  return hipGetLastError();
}

template <typename QT>
hipError_t launch_q(const void* sel_q, const float* sel_w, const void* sel_k,
                    const void* sel_scale, int key_kind, float* scores, int B, int nb, int kpb,
                    int H, int d_idx, hipStream_t stream) {
  switch (key_kind) {
    case kKeyF32:
      return launch_kk<QT, kKeyF32>(sel_q, sel_w, sel_k, sel_scale, scores, B, nb, kpb, H,
                                    d_idx, stream);
    case kKeyBF16:
      return launch_kk<QT, kKeyBF16>(sel_q, sel_w, sel_k, sel_scale, scores, B, nb, kpb, H,
                                     d_idx, stream);
    default:
      return launch_kk<QT, kKeyInt4>(sel_q, sel_w, sel_k, sel_scale, scores, B, nb, kpb, H,
                                     d_idx, stream);
  }
}

}  // namespace

hipError_t launch_select_score(const void* sel_q, bool q_bf16, const float* sel_w,
                               const void* sel_k, const void* sel_k_scale, int key_kind,
                               float* scores, int B, int nb, int kpb, int H, int d_idx,
                               hipStream_t stream) {
  if (q_bf16)
    return launch_q<uint16_t>(sel_q, sel_w, sel_k, sel_k_scale, key_kind, scores, B, nb, kpb,
                              H, d_idx, stream);
  return launch_q<float>(sel_q, sel_w, sel_k, sel_k_scale, key_kind, scores, B, nb, kpb, H,
                         d_idx, stream);
}

}  // namespace spot
