// Prefill variant: tile block scoring and causal block-sparse attention, for one tile
// or a whole sequence cut into tiles. A launch covers B x n_tiles rows; row (b, t) is
// the tile of queries [t*Tq, min((t+1)*Tq, T)) of sequence b, at positions starting at
// q_pos0 + t*Tq, seeing the blocks whose first token is at or before its last query.
//
// Tile scoring (SpotAttention §2.1: one score per query-block x key-block tile, so
// selection runs as a tensor-core matmul; §2.3 per-block maximum). For every selector
// head h, S_h = Qsel_h [Tq x d_idx] . Ksel_h^T [d_idx x blocks] runs on the MFMA units
// (v_mfma_f32_16x16x32_bf16); the epilogue applies ReLU and the per-query weight w[q][h],
// adds the heads, and keeps the maximum over the tile's queries that can see the block.
//
// Attention: one work-group per (HPW row tiles of 16 queries, tile, KV head), G waves;
// each wave computes HPW query heads of one row tile, so the G heads of a KV group share
// every K/V block the work-group stages in LDS (row-major, by direct global-to-LDS
// loads, double-buffered), and each fragment a wave reads back from LDS feeds its HPW
// heads. Per selected block:
//   S' = K . Q^T   (tokens x queries; A = K from LDS, B = Q from registers)
// whose accumulator layout gives each lane 16 scores of one query row. Those become,
// after the online softmax and a bf16 conversion, the A operand of
//   O += P . V     (B = V read with gfx950's transposing LDS load, ds_read_b64_tr_b16,
//                   in the same token order),
// so P never leaves registers; P times a column of ones gives the row sums. Causal and
// L masks are applied per element, only on blocks that cross a row tile's diagonal.
#include "device_common.h"
#include "spot_internal.h"

namespace spot {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBlk = 64;

// ---------------------------------------------------------------- tile scoring
// The tile of launch row r: sequence b, first query row qs, Tq_t queries, first
// position pos0 and nb_vis visible blocks.
struct TileRow {
  int b, qs, Tq_t, pos0, nb_vis;
};
__device__ __forceinline__ TileRow tile_row(int r, int n_tiles, int T, int Tq, int q_pos0,
                                            int block, int nb_stride) {
  TileRow tr;
  tr.b = r / n_tiles;
  tr.qs = (r % n_tiles) * Tq;
  tr.Tq_t = min(Tq, T - tr.qs);
  tr.pos0 = q_pos0 + tr.qs;
  tr.nb_vis = min(nb_stride, (tr.pos0 + tr.Tq_t + block - 1) / block);
  return tr;
}

// Four selector heads (a tile has at most 128 queries): a work-group covers CG groups of
// 16 block columns, its 4 waves taking row tiles wave and wave + 4 of 16 queries. Each
// wave loads the query operands and weights of its row tiles once, then streams only
// keys, 16 blocks at a time, the next group's keys in flight while the current group is
// scored, and the waves combine their column maxima through LDS. With one group per
// work-group every work-group re-reads the tile's 64 KiB of selector queries (d_idx 64);
// with many tiles a work-group takes up to 32 groups (a whole 32K-token row of blocks),
// which cuts that traffic and the work-group count (measured on a 32K prompt in tiles of
// 128: 49 us with 4 groups, 42 with 8, 38 with 16, 37 with 32). 4-bit keys take 16: their
// decode lengthens each group, and the last tile's row is one work-group's serial chain
// (INT4 56 -> 44 us, FP4 46 -> 41; 8 groups: 50 and 45).
constexpr int kScoreMaxCG = 32;
constexpr int kScoreMaxCG4 = 16;

// The B operand of one MFMA k-step of a key row: this lane's 8 elements of d_idx
// (32s + 8kg .. +7), held as loaded and turned into exact bf16 values before use.
// bf16 keys load 16 bytes; 4-bit codes 4 bytes (8 nibbles, even element low); 8-bit
// codes 8 bytes. INT4 codes, FP4 (E2M1) and FP8 (E4M3) values and INT8 codes are all
// exact in bf16, so the product with a bf16 query is exact in the fp32 accumulator and
// the scale is applied to the k-step's dot (per 32-element group) or to the head's dot
// (per tensor), as the format defines the value: code * scale.
template <int KF>
struct KeyRaw {
  typedef typename std::conditional<
      KF == kBF16, bf16x8_t,
      typename std::conditional<KF == kInt4 || KF == kFp4, uint32_t, u32x2_t>::type>::type T;
};

template <int KF>
__device__ __forceinline__ typename KeyRaw<KF>::T load_key_raw(const void* sel_k, size_t row,
                                                              int didx, int s, int kg) {
  // row = index of (b, block, key, head); element offset of this lane's 8 values
  const size_t e = row * didx + s * 32 + kg * 8;
  if constexpr (KF == kBF16) {
    return *reinterpret_cast<const bf16x8_t*>(static_cast<const uint16_t*>(sel_k) + e);
  } else if constexpr (KF == kInt4 || KF == kFp4) {
    return *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(sel_k) + e / 2);
  } else {
    return *reinterpret_cast<const u32x2_t*>(static_cast<const uint8_t*>(sel_k) + e);
  }
}

__device__ __forceinline__ uint16_t bf16_of_small_int(int v) {  // |v| <= 256: exact
  return static_cast<uint16_t>(__float_as_uint(static_cast<float>(v)) >> 16);
}

template <int KF>
__device__ __forceinline__ bf16x8_t decode_key(typename KeyRaw<KF>::T w) {
  if constexpr (KF == kBF16) {
    return w;
  } else if constexpr (KF == kFp4) {
    u32x4_t o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    return __builtin_bit_cast(bf16x8_t, o);
  } else if constexpr (KF == kFp8) {
    u32x4_t o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true));
    return __builtin_bit_cast(bf16x8_t, o);
  } else {
    u32x4_t o;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      int lo, hi;
      if constexpr (KF == kInt4) {  // nibbles 2n (low) and 2n + 1, sign-extended
        lo = static_cast<int>(w << (28 - 8 * n)) >> 28;
        hi = static_cast<int>(w << (24 - 8 * n)) >> 28;
      } else {                      // kInt8: bytes 2n and 2n + 1 of the 8
        const uint32_t word = w[n / 2];
        lo = static_cast<int8_t>((word >> (16 * (n % 2))) & 0xff);
        hi = static_cast<int8_t>((word >> (16 * (n % 2) + 8)) & 0xff);
      }
      o[n] = static_cast<uint32_t>(bf16_of_small_int(lo)) |
             (static_cast<uint32_t>(bf16_of_small_int(hi)) << 16);
    }
    return __builtin_bit_cast(bf16x8_t, o);
  }
}

// The group scale of key row `row` (b, block, key, head), group s, for the group formats
// (INT4: IEEE fp16; FP4: E8M0); 1 otherwise.
template <int KF>
__device__ __forceinline__ float key_group_scale(const void* scale, size_t row, int didx,
                                                 int s) {
  if constexpr (KF == kInt4) {
    return half_bits_to_f(static_cast<const uint16_t*>(scale)[row * (didx / 32) + s]);
  } else if constexpr (KF == kFp4) {
    const uint32_t x = static_cast<const uint8_t*>(scale)[row * (didx / 32) + s];
    return __uint_as_float(x ? (x << 23) : 0x00400000u);  // 2^(x - 127)
  } else {
    return 1.f;
  }
}

template <int KF, int DIDX>
__global__ __launch_bounds__(256) void prefill_score_kernel(
    const uint16_t* __restrict__ sel_q, const float* __restrict__ sel_w,
    const void* __restrict__ sel_k, const void* __restrict__ sel_k_scale,
    float* __restrict__ scores, int T, int Tq, int n_tiles, int q_pos0, int nb_cache,
    int nb_stride, int kpb, int block, int CG) {
  constexpr int H = 4, KS = DIDX / 32, NWV = 4, RPW = 2;
  constexpr bool GROUPS = KF == kInt4 || KF == kFp4;   // one scale per 32 elements
  constexpr bool TENSOR = KF == kInt8 || KF == kFp8;   // one scale for the tensor
  typedef typename KeyRaw<KF>::T Raw;
  __shared__ float colmax[NWV][kScoreMaxCG * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  const TileRow tr = tile_row(blockIdx.y, n_tiles, T, Tq, q_pos0, block, nb_stride);
  const int b = tr.b, Tq_t = tr.Tq_t, pos0 = tr.pos0, nb_vis = tr.nb_vis;
  const int base = blockIdx.x * CG * 16;
  if (base >= nb_vis) return;                       // no visible block here (uniform)
  const int n_cg = min(CG, (nb_vis - base + 15) / 16);
  const int n_rt = (Tq_t + 15) / 16;                // <= NWV * RPW
  const uint16_t* qb = sel_q + ((size_t)b * T + tr.qs) * H * DIDX;
  const float* wb = sel_w + ((size_t)b * T + tr.qs) * H;
  const bool w16 = (reinterpret_cast<uintptr_t>(sel_w) & 15) == 0;
  float tscale = 1.f;
  if constexpr (TENSOR) tscale = *static_cast<const float*>(sel_k_scale);

  // A operands (query row = lane % 16) and weights (queries kg*4 + r) of row tiles
  // wave and wave + NWV
  bf16x8_t qop[RPW][H][KS];
  float wq[RPW][4][H];
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    const int rt = min(wave + u * NWV, n_rt - 1);
    const int qr = min(rt * 16 + col, Tq_t - 1);
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const uint16_t* qp = qb + ((size_t)qr * H + h) * DIDX + kg * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s) qop[u][h][s] = *reinterpret_cast<const bf16x8_t*>(qp + s * 32);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float* wp = wb + (size_t)min(rt * 16 + kg * 4 + r, Tq_t - 1) * H;
      if (w16) {
        const float4 w4 = *reinterpret_cast<const float4*>(wp);
        wq[u][r][0] = w4.x;
        wq[u][r][1] = w4.y;
        wq[u][r][2] = w4.z;
        wq[u][r][3] = w4.w;
      } else {
#pragma unroll
        for (int h = 0; h < H; ++h) wq[u][r][h] = wp[h];
      }
    }
  }
  // B operands of item i = (column group i / kpb, key i % kpb): column = block
  auto load_keys = [&](int i, Raw (&kop)[H][KS], float (&ksc)[H][KS]) {
    const int cg = i / kpb, j = i - cg * kpb;
    const int blk_c = min(base + cg * 16 + col, nb_vis - 1);
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const size_t row = (((size_t)b * nb_cache + blk_c) * kpb + j) * H + h;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kop[h][s] = load_key_raw<KF>(sel_k, row, DIDX, s, kg);
        if constexpr (GROUPS) ksc[h][s] = key_group_scale<KF>(sel_k_scale, row, DIDX, s);
      }
    }
  };
  const int n_items = n_cg * kpb;
  Raw kop[H][KS];
  float ksc[H][KS];
  load_keys(0, kop, ksc);
  float cur = -INFINITY;  // max over (visible query, key) of the current column group
  for (int i = 0; i < n_items; ++i) {  // uniform
    Raw kn[H][KS];
    float kns[H][KS];
    if (i + 1 < n_items) load_keys(i + 1, kn, kns);
    const int cg = i / kpb;
    const int blk = base + cg * 16 + col;
    bf16x8_t kd[H][KS];
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int s = 0; s < KS; ++s) kd[h][s] = decode_key<KF>(kop[h][s]);
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int rt = wave + u * NWV;
      if (rt >= n_rt) break;  // uniform
      floatx4_t tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < H; ++h) {
        floatx4_t c = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GROUPS) {
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const floatx4_t z = {0.f, 0.f, 0.f, 0.f};
            const floatx4_t cs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop[u][h][s], kd[h][s],
                                                                         z, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) c[r] = fmaf(cs[r], ksc[h][s], c[r]);
          }
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop[u][h][s], kd[h][s], c, 0, 0, 0);
          if constexpr (TENSOR) {
#pragma unroll
            for (int r = 0; r < 4; ++r) c[r] *= tscale;
          }
        }
        // c[r] = S_h[query rt*16 + kg*4 + r][column col]
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[r] += wq[u][r][h] * fmaxf(c[r], 0.f);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = rt * 16 + kg * 4 + r;
        const bool vis = qi < Tq_t && (long)blk * block <= (long)pos0 + qi;
        if (vis) cur = fmaxf(cur, tot[r]);
      }
    }
    if (i - cg * kpb == kpb - 1) {  // the group's last key: lanes col, col+16, ... agree
      const float m = xor32_max(xor16_max(cur));
      if (kg == 0) colmax[wave][cg * 16 + col] = m;
      cur = -INFINITY;
    }
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kop[h][s] = kn[h][s];
        if constexpr (GROUPS) ksc[h][s] = kns[h][s];
      }
  }
  __syncthreads();
  if (wave == 0 && kg == 0) {
    for (int cg = 0; cg < n_cg; ++cg) {
      const int blk = base + cg * 16 + col;
      if (blk < nb_vis) {
        float m = colmax[0][cg * 16 + col];
#pragma unroll
        for (int w = 1; w < NWV; ++w) m = fmaxf(m, colmax[w][cg * 16 + col]);
        scores[(size_t)blockIdx.y * nb_stride + blk] = m;
      }
    }
  }
}

// Any H: heads looped at run time (slower path for selector head counts other than 4).
template <int KF, int DIDX>
__global__ __launch_bounds__(64) void prefill_score_kernel_anyh(
    const uint16_t* __restrict__ sel_q, const float* __restrict__ sel_w,
    const void* __restrict__ sel_k, const void* __restrict__ sel_k_scale,
    float* __restrict__ scores, int T, int Tq, int n_tiles, int q_pos0, int nb_cache,
    int nb_stride, int kpb, int H, int block) {
  constexpr int KS = DIDX / 32;
  constexpr bool GROUPS = KF == kInt4 || KF == kFp4;
  constexpr bool TENSOR = KF == kInt8 || KF == kFp8;
  const int lane = threadIdx.x;
  const int col = lane & 15, kg = lane >> 4;
  const TileRow tr = tile_row(blockIdx.y, n_tiles, T, Tq, q_pos0, block, nb_stride);
  const int b = tr.b, Tq_t = tr.Tq_t, pos0 = tr.pos0, nb_vis = tr.nb_vis;
  if (blockIdx.x * 16 >= nb_vis) return;
  const int blk = blockIdx.x * 16 + col;
  const int blk_c = min(blk, nb_vis - 1);
  const int n_rt = (Tq_t + 15) / 16;
  const uint16_t* qb = sel_q + ((size_t)b * T + tr.qs) * H * DIDX;
  const float* wb = sel_w + ((size_t)b * T + tr.qs) * H;
  float tscale = 1.f;
  if constexpr (TENSOR) tscale = *static_cast<const float*>(sel_k_scale);
  float best = -INFINITY;
  for (int j = 0; j < kpb; ++j) {
    for (int rt = 0; rt < n_rt; ++rt) {
      floatx4_t tot = {0.f, 0.f, 0.f, 0.f};
      for (int h = 0; h < H; ++h) {
        const size_t row = (((size_t)b * nb_cache + blk_c) * kpb + j) * H + h;
        const int qr = min(rt * 16 + col, Tq_t - 1);
        const uint16_t* qp = qb + ((size_t)qr * H + h) * DIDX + kg * 8;
        floatx4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8_t kd = decode_key<KF>(load_key_raw<KF>(sel_k, row, DIDX, s, kg));
          const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(qp + s * 32);
          if constexpr (GROUPS) {
            const floatx4_t z = {0.f, 0.f, 0.f, 0.f};
            const floatx4_t cs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kd, z, 0, 0, 0);
            const float sc = key_group_scale<KF>(sel_k_scale, row, DIDX, s);
#pragma unroll
            for (int r = 0; r < 4; ++r) c[r] = fmaf(cs[r], sc, c[r]);
          } else {
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kd, c, 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qi = min(rt * 16 + kg * 4 + r, Tq_t - 1);
          tot[r] += wb[(size_t)qi * H + h] * fmaxf(c[r] * tscale, 0.f);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = rt * 16 + kg * 4 + r;
        const bool vis = qi < Tq_t && (long)blk * block <= (long)pos0 + qi;
        if (vis) best = fmaxf(best, tot[r]);
      }
    }
  }
  best = xor32_max(xor16_max(best));
  if (kg == 0 && blk < nb_vis) scores[(size_t)blockIdx.y * nb_stride + blk] = best;
}

// ---------------------------------------------------------------- attention
constexpr int kMaxPrefillList = 8192;  // longest selected list (32 KiB of LDS at most)
constexpr float kRescaleSlack = 8.f;   // log2 units a row maximum may grow unrescaled
constexpr long kSplitMaxWg = 256;      // one-head grids up to this size split each list in two

// A work-group stages the selected K/V blocks one at a time for RT = HPW row tiles of 16
// queries and the G heads of a KV group: wave w of a group of G waves takes heads
// g*G + (w % (G/HPW))*HPW .. +HPW-1 of row tile w / (G/HPW). Every K or V fragment a wave
// reads from LDS feeds HPW MFMAs, so with HPW = 2 the LDS reads per query and head halve
// (each wave reads the whole 32 KiB block per block). Two work-groups per CU (64 KiB of
// LDS each; about 140 registers with one head per wave, 216 with two). With S = 2 wave
// groups, the groups take alternate blocks of the list and merge their partial softmaxes
// at the end (for grids too small to fill the CUs).
template <int G, int HPW, int S>
__global__ __launch_bounds__(G * S * 64, G * S == 4 ? 2 : 1) void prefill_attn_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, int K_max, uint16_t* __restrict__ out, int Hq,
    int Hkv, int T, int Tq, int n_tiles, int B_rows, int q_pos0, int L, float qscale) {
  constexpr int D = 128;
  constexpr int NT = G * S * 64;
  constexpr int RT = HPW;      // row tiles per work-group
  constexpr int HG = G / HPW;  // waves per row tile
  static_assert(G % HPW == 0, "heads per wave must divide the group");
  // Two block buffers, each a K tile and a V tile of 64 x 128 bf16 (unpadded, chunks
  // swizzled); after the last block buffer A is the output staging area.
  constexpr int TILE = kBlk * D;
  __shared__ __attribute__((aligned(16))) uint16_t bufA[S * 2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t bufB[S * 2 * TILE];
  static_assert(G * HPW * 16 * D <= 2 * TILE, "output staging must fit");
  extern __shared__ int32_t sel_s[];  // the selected list: K_max entries (launch size)

  // XCD-aware order: work-groups are dealt to the 8 XCDs round-robin by linear id, so
  // the row-tile groups of one (tile, KV head) unit get ids of the same residue mod 8
  // and run back to back on one XCD, where the unit's selected blocks stay in its L2.
  const int n_rt = (Tq + 15) / 16;
  const int n_rg = (n_rt + RT - 1) / RT;
  const int lin = blockIdx.x, x = lin & 7, j8 = lin >> 3;
  const int rg = j8 % n_rg;
  const int unit = (j8 / n_rg) * 8 + x;           // (tile row, KV head)
  if (unit >= Hkv * B_rows) return;               // padding of the last group of 8 units
  const int g = unit % Hkv, trow = unit / Hkv;
  const int b = trow / n_tiles, qs = (trow % n_tiles) * Tq;
  const int Tq_t = min(Tq, T - qs);                 // queries of this tile
  const int qg0 = rg * RT * 16;                     // first query row of the work-group
  if (qg0 >= Tq_t) return;                          // past a short last tile (uniform)
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index through readfirstlane, so that the compiler knows everything derived
  // from it (heads, row tile, the per-block full/masked choice) is wave-uniform and
  // branches on it instead of evaluating both sides under a lane mask
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gw = wave % G, split = wave / G;       // wave in its group; the group
  const int h0 = g * G + (gw % HG) * HPW;           // first head of this wave
  const int q0 = qg0 + (gw / HG) * 16;              // its row tile
  const bool active = q0 < Tq_t;                    // uniform per wave
  const int row = lane & 15, kg = lane >> 4;
  const int my_q = q0 + row;                // query row this lane's softmax state tracks
  const int pos0 = q_pos0 + qs;
  const int my_pos = pos0 + my_q;

  // B operand of S' = K.Q^T: column = query row, k = head dim. A negative scale negates
  // q instead (one xor with a wave-uniform mask per register)
  const uint32_t qsign = qscale < 0.f ? 0x80008000u : 0u;
  bf16x8_t qb[HPW][4];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const uint16_t* qp =
        Q + (((size_t)b * Hq + h0 + h) * T + qs + min(my_q, Tq_t - 1)) * D + kg * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(qp + s * 32) ^ qsign;
      qb[h][s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  // scores are scaled into log2 units inside the exponential, by zs > 0 (a zero scale
  // becomes a negligible positive one, so masked scores stay -inf)
  const float zs = fmaxf(fabsf(qscale), 1e-30f);
  // Per head: the running maximum m of query row `row` (same in its 4 lane groups) and
  // O[query (kg*4 + r)][d = dt*16 + row] for dt < 8. Tile dt = 8 multiplies P by a
  // column of ones, so every one of its columns holds the row sums l: the denominator
  // comes from the same bf16 probabilities as the numerator, on the matrix units.
  float m[HPW];
  floatx4_t o[HPW][9];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m[h] = -INFINITY;
#pragma unroll
    for (int dt = 0; dt < 9; ++dt) o[h][dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int cnt = min(max(sel_cnt[trow], 0), K_max);
  const int nbl = (L + kBlk - 1) / kBlk;
  const int last_pos = pos0 + min(qg0 + RT * 16 - 1, Tq_t - 1);  // furthest query
  const uint16_t* Kg = Kc + ((size_t)b * Hkv + g) * (size_t)L * D;
  const uint16_t* Vg = Vc + ((size_t)b * Hkv + g) * (size_t)L * D;

  // the selected list, staged once in LDS (it is read block after block below)
  for (int i = tid; i < cnt; i += NT) sel_s[i] = sel_idx[(size_t)trow * K_max + i];
  __syncthreads();
  // next list entry at or after j whose block exists and is not after the whole
  // work-group's queries
  auto next_block = [&](int j, int& blk) {
    for (; j < cnt; ++j) {
      blk = sel_s[j];
      if (blk >= 0 && blk < nbl && blk * kBlk <= last_pos) return j;
    }
    return cnt;
  };
  // K and V reach LDS by direct global-to-LDS loads (global_load_lds_dwordx4: each lane
  // fetches 16 bytes into its slot of a 1 KiB run), so no registers hold a block in
  // flight. The next block is loaded into one buffer while the other is consumed; one
  // barrier per block both publishes the loaded block and frees the consumed one. The
  // loads are cached ones: the row work-groups of a tile read the same blocks, and
  // adjacent tiles share their recency blocks, so most of them hit in L2.
  //
  // Swizzle: 16-byte chunk c of tile row r sits at chunk c ^ swz(r) of that row, so the
  // 16 rows of a K fragment read and the 8 rows of each half of a transposing V read
  // fall in distinct banks.
  auto swz = [](int r) { return ((r & 7) << 1) | ((r >> 3) & 1); };
  const int ksw = swz(row);                // K fragment rows T*16 + row
  const int vsw = swz(4 * kg + row / 4);   // V rows 32s + 4kg + row/4 (and 16 later)
  // A block wholly inside the cache is addressed as its (wave-uniform) first row plus a
  // per-lane offset fixed for the kernel; only a block crossing L clamps rows to L - 1.
  auto load_block = [&](uint16_t* slot, int blk) {
    const int t0 = blk * kBlk;
    const bool inside = t0 + kBlk <= L;  // uniform
#pragma unroll
    for (int n = 0; n < 16 / G; ++n) {
      const int piece = gw * (16 / G) + n;    // 1 KiB run: tile rows 4*piece .. +3
      const int ch = piece * 64 + lane;       // the LDS chunk this lane fills
      const int r = ch >> 4, c = (ch & 15) ^ swz(ch >> 4);
      const uint16_t* kp;
      const uint16_t* vp;
      if (inside) {
        kp = Kg + (size_t)t0 * D + (r * D + c * 8);
        vp = Vg + (size_t)t0 * D + (r * D + c * 8);
      } else {
        const size_t src = (size_t)min(t0 + r, L - 1) * D + c * 8;
        kp = Kg + src;
        vp = Vg + src;
      }
      __builtin_amdgcn_global_load_lds(
          kp, (__attribute__((address_space(3))) void*)(slot + piece * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          vp, (__attribute__((address_space(3))) void*)(slot + TILE + piece * 512), 16, 0, 0);
    }
  };
  // no block consumed yet by this wave: O and l are still zero, so a first maximum needs
  // no rescale of them (wave-uniform)
  bool fresh = true;
  auto consume = [&](const uint16_t* Ks, int blk) {
    const uint16_t* Vs = Ks + TILE;
    const int t0 = blk * kBlk;
    if (active && t0 <= pos0 + q0 + 15) {  // some token visible to the wave's row tile
      // S'[token][query] for 4 tiles of 16 tokens; each K fragment serves every head
      floatx4_t sc[HPW][4];
#pragma unroll
      for (int T = 0; T < 4; ++T) {
#pragma unroll
        for (int h = 0; h < HPW; ++h) sc[h][T] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        const uint16_t* kp = Ks + (T * 16 + row) * D;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kp + ((kg + 4 * s) ^ ksw) * 8);
#pragma unroll
          for (int h = 0; h < HPW; ++h)
            sc[h][T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[h][s], sc[h][T], 0, 0, 0);
        }
      }
      // sc[h][T][r] = S_h[query row][token T*16 + kg*4 + r], unscaled. One uniform
      // branch for every head: the causal and L masks are computed only for a block that
      // crosses the row tile's diagonal or the end of the cache.
      float bmax[HPW];
#pragma unroll
      for (int h = 0; h < HPW; ++h) bmax[h] = -INFINITY;
      if (!(t0 + kBlk - 1 <= pos0 + q0 && t0 + kBlk <= L)) {
        // token t0 + T*16 + kg*4 + r is visible to this lane's query when T*16 + r <= lim
        const int lim = min(my_pos, L - 1) - t0 - kg * 4;
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool vis = T * 16 + r <= lim;
#pragma unroll
            for (int h = 0; h < HPW; ++h) sc[h][T][r] = vis ? sc[h][T][r] : -INFINITY;
          }
      }
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int r = 0; r < 4; ++r) bmax[h] = fmaxf(bmax[h], sc[h][T][r]);
      }
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        // the block maximum in log2 units (zs > 0, so scaling keeps the order)
        float bm = xor32_max(xor16_max(bmax[h]));
        bm = bm == -INFINITY ? bm : bm * zs;
        // Lazy rescaling: a row's reference maximum m moves only when a block's maximum
        // exceeds it by more than kRescaleSlack (log2 units), so most blocks leave O and
        // l as they are; probabilities stay below 2^kRescaleSlack, well inside bf16 and
        // fp32, and O and l share the reference, so the final O / l is unchanged.
        if (__ballot(bm > m[h] + kRescaleSlack) != 0ull) {  // uniform
          const float mn = bm > m[h] + kRescaleSlack ? bm : m[h];
          const float alpha = mn == m[h] ? 1.f : __builtin_amdgcn_exp2f(m[h] - mn);
          m[h] = mn;
          // rescale O rows kg*4 + r by the alpha of those rows (held by lanes with that row)
          if (!fresh) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float ar = __shfl(alpha, kg * 4 + r, 64);
#pragma unroll
              for (int dt = 0; dt < 9; ++dt) o[h][dt][r] *= ar;
            }
          }
        }
        // v_exp_f32 directly: arguments are at most kRescaleSlack and results below
        // 2^-126 weigh nothing. A row with no visible token yet (m = -inf, so every
        // z = -inf) subtracts 0 instead: its p are 0.
        const float m_s = m[h] == -INFINITY ? 0.f : m[h];
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sc[h][T][r] = __builtin_amdgcn_exp2f(fmaf(sc[h][T][r], zs, -m_s));
      }
      // P as the A operand: k = tokens {32s+4kg..+3} then {32s+16+4kg..+3}; each V
      // fragment serves every head
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8_t pa[HPW];
#pragma unroll
        for (int h = 0; h < HPW; ++h)
          pa[h] = bf16x8_t{(__bf16)sc[h][2 * s][0],     (__bf16)sc[h][2 * s][1],
                           (__bf16)sc[h][2 * s][2],     (__bf16)sc[h][2 * s][3],
                           (__bf16)sc[h][2 * s + 1][0], (__bf16)sc[h][2 * s + 1][1],
                           (__bf16)sc[h][2 * s + 1][2], (__bf16)sc[h][2 * s + 1][3]};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          // lane `row` receives V[32s + 4kg + k][dt*16 + row], k = 0..3, then the same 16
          // tokens later: the token order of pa
          const uint16_t* vp = Vs + (32 * s + 4 * kg + row / 4) * D +
                               ((2 * dt + (row % 4) / 2) ^ vsw) * 8 + 4 * (row & 1);
          const bf16x8_t vb = lds_tr_b_operand(vp, D);
#pragma unroll
          for (int h = 0; h < HPW; ++h)
            o[h][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[h], vb, o[h][dt], 0, 0, 0);
        }
        const bf16x8_t ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                               (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
        for (int h = 0; h < HPW; ++h)
          o[h][8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[h], ones, o[h][8], 0, 0, 0);
      }
      fresh = false;
    }
  };
  // Each set of S blocks (the next S of the list) goes to the S wave groups, one block
  // each: group k loads and consumes entry k of the set in its own slot of the buffer.
  int j = 0;
  auto gather = [&](int (&bl)[S]) {
    bool any = false;
#pragma unroll
    for (int k = 0; k < S; ++k) {
      int blk = 0;
      const int jj = next_block(j, blk);
      bl[k] = jj < cnt ? blk : -1;
      any = any || jj < cnt;
      j = jj < cnt ? jj + 1 : cnt;
    }
    return any;
  };
  int ba[S], bb[S];
  bool has_a = gather(ba);
  if (ba[split] >= 0) load_block(bufA + split * 2 * TILE, ba[split]);
  __syncthreads();
  // Unrolled by two so that every LDS read names the buffer it reads (bufA or bufB) and
  // the compiler need not wait for the other buffer's loads before it.
  while (has_a) {
    const bool has_b = gather(bb);
    if (bb[split] >= 0) load_block(bufB + split * 2 * TILE, bb[split]);
    if (ba[split] >= 0) consume(bufA + split * 2 * TILE, ba[split]);
    __syncthreads();
    if (!has_b) break;
    has_a = gather(ba);
    if (ba[split] >= 0) load_block(bufA + split * 2 * TILE, ba[split]);
    if (bb[split] >= 0) consume(bufB + split * 2 * TILE, bb[split]);
    __syncthreads();
  }
  if constexpr (S == 2) {
    // group 1 hands (m, O, l) to group 0 through buffer B, lane for lane; group 0 merges
    // the two partial softmaxes on the larger reference maximum
    constexpr int NV = HPW * 37;  // floats per lane: m, then 9 tiles x 4
    float* xch = reinterpret_cast<float*>(bufB) + gw * NV * 64 + lane;
    static_assert(G * NV * 64 * 4 <= S * 2 * TILE * 2, "exchange must fit");
    if (split == 1) {
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        xch[(h * 37) * 64] = m[h];
#pragma unroll
        for (int dt = 0; dt < 9; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) xch[(h * 37 + 1 + dt * 4 + r) * 64] = o[h][dt][r];
      }
    }
    __syncthreads();
    if (split == 1) return;
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const float m1 = xch[(h * 37) * 64];
      const float mn = fmaxf(m[h], m1);
      const float a0 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - mn);
      const float a1 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mn);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar0 = __shfl(a0, kg * 4 + r, 64), ar1 = __shfl(a1, kg * 4 + r, 64);
#pragma unroll
        for (int dt = 0; dt < 9; ++dt)
          o[h][dt][r] = o[h][dt][r] * ar0 + xch[(h * 37 + 1 + dt * 4 + r) * 64] * ar1;
      }
    }
  }
  if (!active) return;
  // Normalise, round to bf16 and pass through LDS so that each lane stores whole 16-byte
  // pieces: a head's 16 x 128 output tile is one contiguous 4 KiB run of `out`. The
  // wave's staging region is its own, and every wave is past the loop's last barrier,
  // so no other wave still reads the K/V tiles.
  uint16_t* const st = bufA + wave * (HPW * 16 * D);
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lr = o[h][8][r];  // l of query kg*4 + r
      // the hardware reciprocal (1 ulp): the result is rounded to bf16 below
      const float inv = lr > 0.f ? __builtin_amdgcn_rcpf(lr) : 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        st[(h * 16 + kg * 4 + r) * D + dt * 16 + row] =
            __builtin_bit_cast(uint16_t, (__bf16)(o[h][dt][r] * inv));
    }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    uint16_t* op = out + (((size_t)b * Hq + h0 + h) * T + qs + q0) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = lane + 64 * i;  // 16-byte piece: query c / 16, dims (c % 16) * 8 ..
      if (q0 + c / 16 < Tq_t)
        *reinterpret_cast<u32x4_t*>(op + c * 8) =
            *reinterpret_cast<const u32x4_t*>(&st[(h * 16) * D + c * 8]);
    }
  }
}

template <int KF>
hipError_t launch_prefill_score_kf(const uint16_t* q, const float* sel_w, const void* k,
                                   const void* k_scale, float* scores, int B, int T, int Tq,
                                   int q_pos0, int nb_cache, int nb_stride, int kpb, int H,
                                   int d_idx, int block, hipStream_t stream) {
  const int n_tiles = (T + Tq - 1) / Tq;
  const long groups = (nb_stride + 15) / 16;  // 16-block column groups
  if (H == 4) {
    // several column groups per work-group once there are work-groups to spare
    constexpr int kMaxCG = KF == kInt4 || KF == kFp4 ? kScoreMaxCG4 : kScoreMaxCG;
    const int CG = (long)B * n_tiles * groups >= 2048 ? kMaxCG : 1;
    dim3 grid(static_cast<unsigned>((groups + CG - 1) / CG), B * n_tiles);
#define SPOT_PS4(DI)                                                                         \
  hipLaunchKernelGGL((prefill_score_kernel<KF, DI>), grid, dim3(256), 0, stream, q, sel_w, k, \
                     k_scale, scores, T, Tq, n_tiles, q_pos0, nb_cache, nb_stride, kpb,      \
                     block, CG)
    switch (d_idx) {
      case 32: SPOT_PS4(32); break;
      case 64: SPOT_PS4(64); break;
      default: SPOT_PS4(128); break;
    }
#undef SPOT_PS4
  } else {
    dim3 grid(static_cast<unsigned>(groups), B * n_tiles);
#define SPOT_PSA(DI)                                                                          \
  hipLaunchKernelGGL((prefill_score_kernel_anyh<KF, DI>), grid, dim3(64), 0, stream, q,       \
                     sel_w, k, k_scale, scores, T, Tq, n_tiles, q_pos0, nb_cache, nb_stride, \
                     kpb, H, block)
    switch (d_idx) {
      case 32: SPOT_PSA(32); break;
      case 64: SPOT_PSA(64); break;
      default: SPOT_PSA(128); break;
    }
#undef SPOT_PSA
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_select_score(const void* sel_q, const float* sel_w,
                                       const void* sel_k, const void* sel_k_scale, int k_fmt,
                                       float* scores, int B, int T, int Tq, int q_pos0,
                                       int nb_cache, int nb_stride, int kpb, int H, int d_idx,
                                       int block, hipStream_t stream) {
  const uint16_t* q = static_cast<const uint16_t*>(sel_q);
#define SPOT_PKF(KF)                                                                         \
  return launch_prefill_score_kf<KF>(q, sel_w, sel_k, sel_k_scale, scores, B, T, Tq, q_pos0, \
                                     nb_cache, nb_stride, kpb, H, d_idx, block, stream)
  switch (k_fmt) {
    case kInt4: SPOT_PKF(kInt4);
    case kFp4: SPOT_PKF(kFp4);
    case kInt8: SPOT_PKF(kInt8);
    case kFp8: SPOT_PKF(kFp8);
    default: SPOT_PKF(kBF16);
  }
#undef SPOT_PKF
}

hipError_t launch_prefill_attn(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* sel_idx, const int32_t* sel_cnt, int K_max,
                               void* out, int B, int Hq, int Hkv, int T, int Tq, int q_pos0,
                               int d, int L, float sm_scale, hipStream_t stream) {
  (void)d;
  const int G = Hq / Hkv;
  const int n_tiles = (T + Tq - 1) / Tq;
  const long units = (long)Hkv * B * n_tiles;
  const size_t lds_list = (size_t)K_max * sizeof(int32_t);  // K_max <= kMaxPrefillList
  const int n_rt = (Tq + 15) / 16;
  const float qscale = sm_scale * kLog2e;
  const uint16_t* Qp = static_cast<const uint16_t*>(q);
  const uint16_t* Kp = static_cast<const uint16_t*>(k_cache);
  const uint16_t* Vp = static_cast<const uint16_t*>(v_cache);
  uint16_t* Op = static_cast<uint16_t*>(out);
  // grid: units in groups of 8 (one per XCD) x groups of HPW row tiles
#define SPOT_PF(GG, HPW, SS)                                                                \
  do {                                                                                      \
    const dim3 grid(static_cast<unsigned>((units + 7) / 8 * 8 * ((n_rt + HPW - 1) / HPW))); \
    (void)hipFuncSetAttribute(                                                              \
        reinterpret_cast<const void*>(&prefill_attn_kernel<GG, HPW, SS>),                  \
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_list);                         \
    hipLaunchKernelGGL((prefill_attn_kernel<GG, HPW, SS>), grid, dim3(GG * SS * 64),        \
                       lds_list, stream, Qp, Kp, Vp, sel_idx, sel_cnt, K_max, Op, Hq, Hkv, T, \
                       Tq, n_tiles, B * n_tiles, q_pos0, L, qscale);                        \
  } while (0)
  // Two heads per wave (half the LDS reads per head) pay once the one-head grid has
  // work-groups to spare -- at least 1024, four per CU -- and the row tiles pair up
  // (an odd count leaves one wave of the last pair idle). Measured on the 32/8-head,
  // 128-query-tile layer: 10-20 % faster from 1024 work-groups up, 8 % slower at 512
  // and 40 % slower for a lone tile. A grid that fits the CUs once over (one work-group
  // each) instead splits every list between two wave groups per work-group, which halves
  // the chain of blocks each wave runs (a lone 128-query tile: 3 % faster, 256
  // work-groups: 7 %; at 512 work-groups, 128 KiB of LDS per work-group costs more).
  const bool two_heads = G == 4 && (n_rt % 2 == 0 || n_rt >= 7) && units * n_rt >= 1024;
  switch (G) {
    case 1: SPOT_PF(1, 1, 1); break;
    case 2: SPOT_PF(2, 1, 1); break;
    case 4:
      if (two_heads) SPOT_PF(4, 2, 1);
      else if (units * n_rt <= kSplitMaxWg) SPOT_PF(4, 1, 2);
      else SPOT_PF(4, 1, 1);
      break;
    default: SPOT_PF(8, 1, 1); break;
  }
#undef SPOT_PF
  return hipGetLastError();
}

}  // namespace spot
