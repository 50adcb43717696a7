// Host-side launchers implemented by the kernel translation units and called by the
// C ABI after argument validation. Each returns hipSuccess or the launch error.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spot.h"

namespace spot {

// Selector element formats (the values of the C ABI's spot_dtype codes).
enum Fmt { kF32 = 0, kBF16 = 1, kInt4 = 2, kInt8 = 3, kFp8 = 4, kFp4 = 5 };

hipError_t launch_select_score(const void* sel_q, int q_fmt, const void* sel_q_scale,
                               const float* sel_w, const void* sel_k, const void* sel_k_scale,
                               int k_fmt, float* scores, int B, int nb, int kpb, int H,
                               int d_idx, hipStream_t stream);

hipError_t launch_quantize_selector(const void* src, bool src_bf16, int fmt, void* codes,
                                    void* scales, const float* tensor_scale, long n_groups,
                                    hipStream_t stream);

hipError_t launch_prefill_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                                      float* sel_mass, int B, int T, int Tq, int q_pos0,
                                      int block, int nb_stride, float p, int K_min, int K_max,
                                      int n_sink, int n_rec, hipStream_t stream);

hipError_t launch_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                              float* sel_mass, int B, int nb, float p, int K_min, int K_max,
                              int n_sink, int n_rec, hipStream_t stream);

// Split geometry of the decode attention (attn_plan.cpp): blocks per run and the number
// of runs per (query, KV head); a pure function of the sizes so the workspace bound holds.
constexpr int kFlatMaxB = 64;  // bf16 batches up to this size cut runs across queries
struct AttnSplit {
  int blocks_per_split;
  int nsplit;
  bool flat;  // runs cut across queries (the MFMA path at small batch)
  int nslot;  // partial-result slots per (query, head)
  int waves;  // waves per work-group of the MFMA path: 8 (one chunk each) or 4
};
AttnSplit attn_split_plan(int B, int Hkv, int K_max, int block, bool bf16_fast_path);
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int d, int K_max, int block, bool bf16);

// Size of the per-GPU device array behind spot_sparse_attn_noalloc, and its device
// address on the stream's GPU (looked up on the first call for that GPU).
constexpr size_t kNoallocScratchBytes = SPOT_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

hipError_t launch_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                              bool bf16, const int32_t* sel_idx, const int32_t* sel_cnt,
                              int K_max, void* out, void* workspace, int B, int Hq, int Hkv,
                              int d, int L, int block, float sm_scale, hipStream_t stream);

// Prefill: a sequence of T query rows per batch element, cut into tiles of Tq rows
// (T == Tq: one tile); score rows are [B][n_tiles][nb_stride].
hipError_t launch_prefill_select_score(const void* sel_q, const float* sel_w,
                                       const void* sel_k, const void* sel_k_scale, int k_fmt,
                                       float* scores, int B, int T, int Tq, int q_pos0,
                                       int nb_cache, int nb_stride, int kpb, int H, int d_idx,
                                       int block, hipStream_t stream);

hipError_t launch_prefill_attn(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* sel_idx, const int32_t* sel_cnt, int K_max,
                               void* out, int B, int Hq, int Hkv, int T, int Tq, int q_pos0,
                               int d, int L, float sm_scale, hipStream_t stream);

}  // namespace spot
