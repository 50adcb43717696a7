// C ABI of libspot: argument validation and dispatch to the HIP launchers.
// Every check happens on the host before anything is enqueued; no HIP call is made
// for an invalid or unsupported argument set.
#include <math.h>
#include <stdint.h>

#include "../../include/spot.h"
#include "spot_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
int from_hip(hipError_t e) {
  if (e == hipErrorNotSupported) return SPOT_ERR_UNSUPPORTED;
  return e == hipSuccess ? SPOT_OK : SPOT_ERR_DEVICE;
}

constexpr int kMaxGrid = 65535;  // grid.y / grid.z limit used by the launchers

// A selector tensor in one of the spot_dtype formats with its scale array: the format
// must be known, quantised formats need their scale (aligned to its element) and the
// group formats need d_idx % 32 == 0; fp32/bf16 take no scale.
int check_format(int fmt, const void* scale, int d_idx) {
  switch (fmt) {
    case SPOT_F32:
    case SPOT_BF16:
      return scale ? SPOT_ERR_INVALID : SPOT_OK;
    case SPOT_INT8:
    case SPOT_FP8_E4M3:
      return scale && aligned(scale, 4) ? SPOT_OK : SPOT_ERR_INVALID;
    case SPOT_INT4_G32:
      return scale && aligned(scale, 2) && d_idx % 32 == 0 ? SPOT_OK : SPOT_ERR_INVALID;
    case SPOT_FP4_E2M1_G32:
      return scale && d_idx % 32 == 0 ? SPOT_OK : SPOT_ERR_INVALID;
    default:
      return SPOT_ERR_INVALID;
  }
}

// elements of d_idx one 16-byte load of a key row holds, per format
int key_chunk(int fmt) {
  switch (fmt) {
    case SPOT_INT8:
    case SPOT_FP8_E4M3: return 16;
    case SPOT_INT4_G32:
    case SPOT_FP4_E2M1_G32: return 32;
    default: return 8;
  }
}

// Common validation of a selector description; returns SPOT_OK or an error.
int check_selector(const void* sel_q, int q_dtype, const void* sel_q_scale, const float* sel_w,
                   const void* sel_k, const void* sel_k_scale, int k_dtype, int H_idx,
                   int d_idx, int kpb) {
  if (!sel_q || !sel_w || !sel_k) return SPOT_ERR_INVALID;
  if (H_idx <= 0 || d_idx <= 0 || kpb <= 0) return SPOT_ERR_INVALID;
  if (!aligned(sel_q, 16) || !aligned(sel_w, 4) || !aligned(sel_k, 16)) return SPOT_ERR_INVALID;
  if (check_format(q_dtype, sel_q_scale, d_idx) != SPOT_OK) return SPOT_ERR_INVALID;
  if (check_format(k_dtype, sel_k_scale, d_idx) != SPOT_OK) return SPOT_ERR_INVALID;
  if (d_idx != 32 && d_idx != 64 && d_idx != 128) return SPOT_ERR_UNSUPPORTED;
  const int lpr = H_idx * (d_idx / key_chunk(k_dtype));
  if (!pow2(H_idx) || lpr > 64) return SPOT_ERR_UNSUPPORTED;
  return SPOT_OK;
}

// The attention shapes the library has kernels for (after the argument checks).
int attn_support(int Hq, int Hkv, int d, int block) {
  const int G = Hq / Hkv;
  if (d != 64 && d != 128) return SPOT_ERR_UNSUPPORTED;
  if (block != 16 && block != 32 && block != 64 && block != 128) return SPOT_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return SPOT_ERR_UNSUPPORTED;
  return SPOT_OK;
}

// Argument checks shared by spot_sparse_attn and spot_sparse_attn_noalloc (the
// workspace pointer and size are checked by the caller).
int check_sparse_attn(const void* q, const void* k_cache, const void* v_cache, int kv_dtype,
                      const int32_t* sel_idx, const int32_t* sel_cnt, int K_max,
                      const void* out, int B, int Hq, int Hkv, int d, int L, int block,
                      float sm_scale) {
  if (!q || !k_cache || !v_cache || !sel_idx || !sel_cnt || !out) return SPOT_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(sel_idx, 4) || !aligned(sel_cnt, 4))
    return SPOT_ERR_INVALID;
  if (kv_dtype != SPOT_F32 && kv_dtype != SPOT_BF16) return SPOT_ERR_INVALID;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || L <= 0 || block <= 0 || K_max <= 0)
    return SPOT_ERR_INVALID;
  if (Hq % Hkv != 0 || !isfinite(sm_scale)) return SPOT_ERR_INVALID;
  const int sup = attn_support(Hq, Hkv, d, block);
  if (sup != SPOT_OK) return sup;
  if (B > kMaxGrid || Hkv > kMaxGrid || (long)B * Hq > 2147483647L) return SPOT_ERR_UNSUPPORTED;
  return SPOT_OK;
}

}  // namespace

extern "C" {

int spot_abi_version(void) { return 3; }

const char* spot_status_string(int status) {
  switch (status) {
    case SPOT_OK: return "SPOT_OK";
    case SPOT_ERR_INVALID: return "SPOT_ERR_INVALID: invalid argument";
    case SPOT_ERR_UNSUPPORTED: return "SPOT_ERR_UNSUPPORTED: no kernel for this combination";
    case SPOT_ERR_DEVICE: return "SPOT_ERR_DEVICE: the HIP runtime refused a launch";
    default: return "unknown spot status";
  }
}

int spot_select_score(const void* sel_q, int q_dtype, const void* sel_q_scale,
                      const float* sel_w, const void* sel_k, const void* sel_k_scale,
                      int k_dtype, float* scores, int B, int nb, int kpb, int H_idx, int d_idx,
                      void* stream) {
  if (B <= 0 || nb <= 0 || !scores || !aligned(scores, 4)) return SPOT_ERR_INVALID;
  const int c = check_selector(sel_q, q_dtype, sel_q_scale, sel_w, sel_k, sel_k_scale, k_dtype,
                               H_idx, d_idx, kpb);
  if (c != SPOT_OK) return c;
  if (B > kMaxGrid) return SPOT_ERR_UNSUPPORTED;
  return from_hip(spot::launch_select_score(sel_q, q_dtype, sel_q_scale, sel_w, sel_k,
                                            sel_k_scale, k_dtype, scores, B, nb, kpb, H_idx,
                                            d_idx, as_stream(stream)));
}

int spot_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt, float* sel_mass,
                     int B, int nb, float p, int K_min, int K_max, int n_sink, int n_rec,
                     void* stream) {
  if (!scores || !sel_idx || !sel_cnt) return SPOT_ERR_INVALID;
  if (!aligned(scores, 4) || !aligned(sel_idx, 4) || !aligned(sel_cnt, 4) ||
      (sel_mass && !aligned(sel_mass, 4)))
    return SPOT_ERR_INVALID;
  if (B <= 0 || nb <= 0 || K_max <= 0) return SPOT_ERR_INVALID;
  if (!isfinite(p) || n_sink < 0 || n_rec < 0 || K_min < 0) return SPOT_ERR_INVALID;
  const int rs = n_sink < nb ? n_sink : nb;
  const int rr = n_rec < nb ? n_rec : nb;
  const int r = rs + rr < nb ? rs + rr : nb;
  if (K_max < r) return SPOT_ERR_INVALID;
  if (nb > 16384) return SPOT_ERR_UNSUPPORTED;
  if (B > 2147483647 / 2) return SPOT_ERR_UNSUPPORTED;
  return from_hip(spot::launch_select_topp(scores, sel_idx, sel_cnt, sel_mass, B, nb, p, K_min,
                                           K_max, n_sink, n_rec, as_stream(stream)));
}

int spot_quantize_selector(const void* src, int src_dtype, int n_rows, int row_len, int fmt,
                           void* codes, void* scales, const float* tensor_scale,
                           void* stream) {
  if (!src || !codes || n_rows <= 0 || row_len <= 0 || row_len % 32 != 0)
    return SPOT_ERR_INVALID;
  if (src_dtype != SPOT_F32 && src_dtype != SPOT_BF16) return SPOT_ERR_INVALID;
  if (!aligned(src, 16) || !aligned(codes, 16)) return SPOT_ERR_INVALID;
  switch (fmt) {
    case SPOT_INT4_G32:
      if (!scales || !aligned(scales, 2) || tensor_scale) return SPOT_ERR_INVALID;
      break;
    case SPOT_FP4_E2M1_G32:
      if (!scales || tensor_scale) return SPOT_ERR_INVALID;
      break;
    case SPOT_INT8:
    case SPOT_FP8_E4M3:
      if (scales || !tensor_scale || !aligned(tensor_scale, 4)) return SPOT_ERR_INVALID;
      break;
    default:
      return SPOT_ERR_INVALID;
  }
  const long n_groups = (long)n_rows * (row_len / 32);
  if (n_groups > 255L * 2147483647L) return SPOT_ERR_UNSUPPORTED;
  return from_hip(spot::launch_quantize_selector(src, src_dtype == SPOT_BF16, fmt, codes,
                                                 scales, tensor_scale, n_groups,
                                                 as_stream(stream)));
}

size_t spot_sparse_attn_workspace_bytes(int B, int Hq, int Hkv, int d, int K_max, int block,
                                        int kv_dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || K_max <= 0 || block <= 0) return 0;
  if (Hq % Hkv != 0 || (kv_dtype != SPOT_F32 && kv_dtype != SPOT_BF16)) return 0;
  if (attn_support(Hq, Hkv, d, block) != SPOT_OK) return 0;
  return spot::attn_workspace_bytes(B, Hq, Hkv, d, K_max, block, kv_dtype == SPOT_BF16);
}

int spot_sparse_attn(const void* q, const void* k_cache, const void* v_cache, int kv_dtype,
                     const int32_t* sel_idx, const int32_t* sel_cnt, int K_max, void* out,
                     void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int d,
                     int L, int block, float sm_scale, void* stream) {
  const int c = check_sparse_attn(q, k_cache, v_cache, kv_dtype, sel_idx, sel_cnt, K_max, out,
                                  B, Hq, Hkv, d, L, block, sm_scale);
  if (c != SPOT_OK) return c;
  if (!workspace || !aligned(workspace, 256)) return SPOT_ERR_INVALID;
  if (workspace_bytes <
      spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, K_max, block, kv_dtype))
    return SPOT_ERR_INVALID;
  return from_hip(spot::launch_sparse_attn(q, k_cache, v_cache, kv_dtype == SPOT_BF16, sel_idx,
                                           sel_cnt, K_max, out, workspace, B, Hq, Hkv, d, L,
                                           block, sm_scale, as_stream(stream)));
}

int spot_sparse_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                             int kv_dtype, const int32_t* sel_idx, const int32_t* sel_cnt,
                             int K_max, void* out, int B, int Hq, int Hkv, int d, int L,
                             int block, float sm_scale, void* stream) {
  const int c = check_sparse_attn(q, k_cache, v_cache, kv_dtype, sel_idx, sel_cnt, K_max, out,
                                  B, Hq, Hkv, d, L, block, sm_scale);
  if (c != SPOT_OK) return c;
  if (spot_sparse_attn_workspace_bytes(B, Hq, Hkv, d, K_max, block, kv_dtype) >
      spot::kNoallocScratchBytes)
    return SPOT_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const hipError_t e = spot::noalloc_scratch(as_stream(stream), &ws);
  if (e != hipSuccess || !ws) return SPOT_ERR_DEVICE;
  return from_hip(spot::launch_sparse_attn(q, k_cache, v_cache, kv_dtype == SPOT_BF16, sel_idx,
                                           sel_cnt, K_max, out, ws, B, Hq, Hkv, d, L, block,
                                           sm_scale, as_stream(stream)));
}

int spot_prefill_select_score(const void* sel_q, int q_dtype, const float* sel_w,
                              const void* sel_k, const void* sel_k_scale, int k_dtype,
                              float* scores, int B, int T, int Tq, int q_pos0, int nb_cache,
                              int kpb, int H_idx, int d_idx, int block, void* stream) {
  if (B <= 0 || T <= 0 || Tq <= 0 || q_pos0 < 0 || nb_cache <= 0 || block <= 0)
    return SPOT_ERR_INVALID;
  if (!scores || !aligned(scores, 4)) return SPOT_ERR_INVALID;
  const int c = check_selector(sel_q, q_dtype, nullptr, sel_w, sel_k, sel_k_scale, k_dtype,
                               H_idx, d_idx, kpb);
  if (c != SPOT_OK) return c;
  if ((long)q_pos0 + T > 2147483647L) return SPOT_ERR_INVALID;  // positions are int
  const long nb_seq = ((long)q_pos0 + T + block - 1) / block;
  if (nb_seq > nb_cache) return SPOT_ERR_INVALID;
  if (q_dtype != SPOT_BF16 || k_dtype == SPOT_F32) return SPOT_ERR_UNSUPPORTED;
  const long rows = (long)B * ((T + Tq - 1) / Tq);
  if (Tq > 128 || rows > kMaxGrid) return SPOT_ERR_UNSUPPORTED;
  return from_hip(spot::launch_prefill_select_score(sel_q, sel_w, sel_k, sel_k_scale, k_dtype,
                                                    scores, B, T, Tq, q_pos0, nb_cache,
                                                    (int)nb_seq, kpb, H_idx, d_idx, block,
                                                    as_stream(stream)));
}

int spot_prefill_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                             float* sel_mass, int B, int T, int Tq, int q_pos0, int block,
                             float p, int K_min, int K_max, int n_sink, int n_rec,
                             void* stream) {
  if (!scores || !sel_idx || !sel_cnt) return SPOT_ERR_INVALID;
  if (!aligned(scores, 4) || !aligned(sel_idx, 4) || !aligned(sel_cnt, 4) ||
      (sel_mass && !aligned(sel_mass, 4)))
    return SPOT_ERR_INVALID;
  if (B <= 0 || T <= 0 || Tq <= 0 || q_pos0 < 0 || block <= 0 || K_max <= 0)
    return SPOT_ERR_INVALID;
  if (!isfinite(p) || n_sink < 0 || n_rec < 0 || K_min < 0) return SPOT_ERR_INVALID;
  if ((long)q_pos0 + T > 2147483647L) return SPOT_ERR_INVALID;  // positions are int
  const long nb_seq = ((long)q_pos0 + T + block - 1) / block;
  if (nb_seq > 16384) return SPOT_ERR_UNSUPPORTED;
  const int nb = (int)nb_seq;
  const int rs = n_sink < nb ? n_sink : nb;
  const int rr = n_rec < nb ? n_rec : nb;
  const int r = rs + rr < nb ? rs + rr : nb;  // the largest reserved set of any tile
  if (K_max < r) return SPOT_ERR_INVALID;
  const long rows = (long)B * ((T + Tq - 1) / Tq);
  if (rows > 2147483647L / 2) return SPOT_ERR_UNSUPPORTED;
  return from_hip(spot::launch_prefill_select_topp(scores, sel_idx, sel_cnt, sel_mass, B, T, Tq,
                                                   q_pos0, block, nb, p, K_min, K_max, n_sink,
                                                   n_rec, as_stream(stream)));
}

int spot_prefill_attn(const void* q, const void* k_cache, const void* v_cache, int kv_dtype,
                      const int32_t* sel_idx, const int32_t* sel_cnt, int K_max, void* out,
                      int B, int Hq, int Hkv, int T, int Tq, int q_pos0, int d, int L,
                      int block, float sm_scale, void* stream) {
  if (!q || !k_cache || !v_cache || !sel_idx || !sel_cnt || !out) return SPOT_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(sel_idx, 4) || !aligned(sel_cnt, 4))
    return SPOT_ERR_INVALID;
  if (kv_dtype != SPOT_F32 && kv_dtype != SPOT_BF16) return SPOT_ERR_INVALID;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || Tq <= 0 || q_pos0 < 0 || d <= 0 || L <= 0 ||
      block <= 0 || K_max <= 0)
    return SPOT_ERR_INVALID;
  if (Hq % Hkv != 0 || !isfinite(sm_scale)) return SPOT_ERR_INVALID;
  if ((long)q_pos0 + T > L) return SPOT_ERR_INVALID;
  const int G = Hq / Hkv;
  if (kv_dtype != SPOT_BF16 || d != 128 || block != 64 || Tq > 128 || K_max > 8192)
    return SPOT_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return SPOT_ERR_UNSUPPORTED;
  const long rows = (long)B * ((T + Tq - 1) / Tq);
  if (rows > kMaxGrid || Hkv > kMaxGrid) return SPOT_ERR_UNSUPPORTED;
  return from_hip(spot::launch_prefill_attn(q, k_cache, v_cache, sel_idx, sel_cnt, K_max, out, B,
                                            Hq, Hkv, T, Tq, q_pos0, d, L, sm_scale,
                                            as_stream(stream)));
}

}  // extern "C"
