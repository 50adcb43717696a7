// Split plan of the decode attention (host code): how the selected-block lists are cut
// into runs, one work-group each, and how many partial-result slots a (query, head)
// needs. A pure function of the sizes, shared by the launcher and the workspace size.
#include <algorithm>

#include "spot_internal.h"

namespace spot {

AttnSplit attn_split_plan(int B, int Hkv, int K_max, int block, bool bf16_fast_path) {
  AttnSplit sp;
  const long units = (long)B * Hkv;
  if (!bf16_fast_path) {
    // one wave per run: 4 blocks, or longer runs so that a row has at most 64 of them
    sp.blocks_per_split = K_max > 256 ? (int)(((long)K_max + 63) / 64) : 4;
  } else {
    // the longest run (<= 4096 tokens, i.e. 64 chunks: at most 16 per wave, and at
    // most 64 list entries per wave) that still gives >= 256 work-groups
    int bps = 0;
    for (int tokens = 4096; tokens >= 256 && bps == 0; tokens >>= 1) {
      const int c = tokens / block;
      if (units * (((long)K_max + c - 1) / c) >= 256) bps = c;
    }
    sp.blocks_per_split = bps > 0 ? bps : 256 / block;
  }
  sp.nsplit = (int)(((long)K_max + sp.blocks_per_split - 1) / sp.blocks_per_split);
  // Runs across queries (MFMA path, 2 <= B <= kFlatMaxB): a query's runs fill its slots
  // from 0, at most nslot of them. nsplit * B slots would let one long query take every
  // work-group of the batch; max(nsplit, 32) keeps that freedom at small batches (it is
  // nsplit * B up to batch 8 at 256 work-groups) and bounds the workspace at large ones.
  // Runs of at most 8 64-token chunks (few queries and KV heads, e.g. one query at 128K)
  // go to 8 waves of one chunk each, K and V loaded together, instead of 4 waves of two
  // chunks with the next K prefetched: every wave has one load latency instead of two.
  sp.waves = bf16_fast_path && (long)sp.blocks_per_split * block <= 8 * 64 ? 8 : 4;
  sp.flat = bf16_fast_path && B >= 2 && B <= kFlatMaxB;
  sp.nslot = sp.flat ? (int)std::min<long>((long)sp.nsplit * B, std::max(sp.nsplit, 32))
                     : sp.nsplit;
  return sp;
}

size_t attn_workspace_bytes(int B, int Hq, int Hkv, int d, int K_max, int block, bool bf16) {
  // fp32 partial results and (m, l) per slot: nslot slots per (query, head)
  const AttnSplit sp = attn_split_plan(B, Hkv, K_max, block, bf16);
  return (size_t)B * Hq * (size_t)sp.nslot * ((size_t)d + 2) * sizeof(float);
}

}  // namespace spot
