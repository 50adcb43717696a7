// Decode attention over the selected KV blocks (SpotAttention §2.3: the layer attends
// only to keys in blocks of S_q, one S_q per query shared by every head).
//
// Split-K: the selected-block lists are cut into runs; a work-group reduces one run with
// an online softmax for the G query heads that share a KV head (GQA) and stores
// (m, l, acc) per head in a slot of that query. The MFMA path at batch 2..64 cuts the
// lists of all queries, concatenated, into equal runs (a run may end one query's list
// and start the next one's, one partial each), so queries that select very different
// numbers of blocks still keep every work-group equally busy; otherwise each
// (query, KV head) gets the same number of runs, cut from that query's own count (runs
// past its end store an empty partial). A second kernel then merges the slots of every
// (query, head) (attn_merge32 for up to 32 slots, attn_combine above that; both
// deterministic). Merging inside the run kernel, in the last work-group of each
// (query, KV head) to finish, was measured twice and is slower on this multi-XCD part:
// with agent-scope release/acquire (an L2 writeback plus invalidate per work-group) the
// 128K batch-8 call took 108 us instead of 84 and the 1024-block static top-K call 593
// instead of 334; with write-through partials, one atomic ticket per work-group and the
// partials read back past L2 it took 90 instead of ~87 us per batch-8 call and 25.4
// instead of ~19 at batch 1 (the last work-group's chain of round trips costs more than
// the kernel boundary).
//
// Block sizes 16, 32, 64 and 128 tokens. The unit of work of a wave is a 64-token
// chunk made of four 16-token tiles, each with its own start token: the four tiles of
// one 64-token block, two 32-token blocks, four 16-token blocks (the paper's page
// size) or half a 128-token block. Run lengths are chosen in tokens, so every block
// size moves the same bytes per work-group.
//
// HBM-bound (about 4 flop per byte in bf16 with G = 4). Two run kernels:
//  * attn_mfma (bf16, d in {64,128}): each wave owns whole 64-token chunks, and both
//    products run on the MFMA units (v_mfma_f32_16x16x32_bf16, the G heads padded to
//    16). S' = K.Q^T (tokens x heads): every lane loads 16 contiguous bytes of a K row
//    straight into the A-operand layout, no LDS staging. The accumulator layout leaves
//    each lane 16 scores of one head, so the online softmax reduces across four lanes
//    and the probabilities, rounded to bf16, are already the A operand of O += P.V;
//    V goes to a per-wave LDS tile (coalesced 16-byte row loads) and comes back as the
//    B operand through gfx950's transposing LDS read. K and V are read once, so their
//    loads are non-temporal (measured: ~7% more HBM throughput on this random-block
//    gather than cached loads), and each wave loads the next chunk's K while it
//    consumes the current one (~5% more). Runs of at most 8 chunks (one query at 128K:
//    8 KV heads x 32 runs) use 8 waves of one chunk each instead, K and V issued
//    together (206 registers, two waves per SIMD): one exposed load latency per wave
//    instead of two (batch-1 split kernel 14.8 -> 14.2 us).
//  * attn_generic (fp32 or bf16, any supported shape): one wave per run;
//    lane = token for q.K^T (64 tokens of a block at a time), lane = head dim for P.V,
//    all in fp32.
// Scores are kept in the log2 domain: z = (q.k) * sm_scale * log2(e), p = 2^(z - m).
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "spot_internal.h"

namespace spot {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 64;  // tokens a wave consumes at a time (four 16-token tiles)

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t x) { return bf16_to_f(x); }
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = f_to_bf16_rne(v); }

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Partial results are stored with agent-scope (relaxed atomic) stores, which write
// through the XCD's L2 to the device-coherent level: the kernel's end then has fewer
// dirty L2 lines to write back before the merge kernel may start (measured: 0.1 us
// less per 128K call at batch 1 and 8).
__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_partial(float2* p, float2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The run result of this work-group (per head: max m, sum l, unnormalised acc[D]), held
// in LDS, stored as the run's partial result for the merge. `last` marks a head's
// last partial: its l is stored as -l - 1 (a real l is >= 0), and the merge stops after
// it.
template <int D, int G, int NT>
__device__ void store_run(const float (&racc)[G][D], const float (&rm)[G], const float (&rl)[G],
                          size_t base, int nslot, float* __restrict__ ws_acc,
                          float2* __restrict__ ws_ml, bool last = false) {
  for (int o = threadIdx.x; o < G * D; o += NT) {
    const int h = o / D, dd = o % D;
    const size_t idx = base + (size_t)h * nslot;
    store_partial(&ws_acc[idx * D + dd], racc[h][dd]);
    if (dd == 0) store_partial(&ws_ml[idx], make_float2(rm[h], last ? -rl[h] - 1.f : rl[h]));
  }
}

// Partial-result slots: head hq of query b owns nslot consecutive slots from
// (b * Hq + hq) * nslot; a work-group writes slot `slot` of its G heads, so `base` is
// (b * Hq + g * G) * nslot + slot and head h of the group is base + h * nslot.
__host__ __device__ inline size_t slot_base(int b, int g, int G, int Hq, int nslot, int slot) {
  return ((size_t)b * Hq + (size_t)g * G) * nslot + slot;
}

// A run with nothing to merge: an empty partial (m = -inf, l = 0).
template <int G>
__device__ void store_empty_run(size_t base, int nslot, float2* __restrict__ ws_ml) {
  if (threadIdx.x < G)
    store_partial(&ws_ml[base + (size_t)threadIdx.x * nslot], make_float2(-INFINITY, 0.f));
}

// An empty last partial (m = -inf, l = 0 stored as -1): a query with no entry, or the
// empty final run of a query.
template <int G>
__device__ void store_end_marker(size_t base, int nslot, float2* __restrict__ ws_ml) {
  if (threadIdx.x < G)
    store_partial(&ws_ml[base + (size_t)threadIdx.x * nslot], make_float2(-INFINITY, -1.f));
}

// ---------------------------------------------------------------- generic pass 1
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void attn_generic(
    const T* __restrict__ q, const T* __restrict__ Kc, const T* __restrict__ Vc,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt, int K_max,
    float* __restrict__ ws_acc, float2* __restrict__ ws_ml, int Hq, int Hkv, int L,
    float qscale, int block, int bps, int nsplit) {
  constexpr int DPL = D / 64;  // head dims per lane in P.V
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int cnt = min(max(sel_cnt[b], 0), K_max);
  const int j0 = split * bps;
  if (j0 >= cnt) {
    store_empty_run<G>(slot_base(b, g, G, Hq, nsplit, split), nsplit, ws_ml);
    return;
  }
  const int j1 = min(j0 + bps, cnt);
  const int lane = threadIdx.x;
  __shared__ float qs[G][D];
  __shared__ float ps[kChunk][G];
  for (int i = lane; i < G * D; i += 64) {
    const int h = i / D, dd = i % D;
    qs[h][dd] = to_f(q[((size_t)b * Hq + g * G + h) * D + dd]) * qscale;
  }
  __syncthreads();
  float m[G], l[G], acc[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) acc[h][c] = 0.f;
  }
  const int nbl = (L + block - 1) / block;
  const T* Kg = Kc + ((size_t)b * Hkv + g) * (size_t)L * D;
  const T* Vg = Vc + ((size_t)b * Hkv + g) * (size_t)L * D;
  for (int j = j0; j < j1; ++j) {
    const int blk = sel_idx[(size_t)b * K_max + j];
    if (blk < 0 || blk >= nbl) continue;
    // 64 tokens of the block at a time; at least one of them is < L
    for (int c0 = 0; c0 < block && blk * block + c0 < L; c0 += kChunk) {
    const int t0 = blk * block + c0;
    const int ntok = min(min(kChunk, block - c0), L - t0);
    const int tok = t0 + lane;
    const bool tv = lane < ntok;
    const T* kr = Kg + (size_t)(tv ? tok : L - 1) * D;
    float z[G];
#pragma unroll
    for (int h = 0; h < G; ++h) z[h] = 0.f;
#pragma unroll 4
    for (int d0 = 0; d0 < D; d0 += 8) {
      float kv[8];
      load8(kr + d0, kv);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int n = 0; n < 8; ++n) z[h] = fmaf(qs[h][d0 + n], kv[n], z[h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float zz = tv ? z[h] : -INFINITY;
      const float mn = fmaxf(m[h], group_max<64>(zz));
      const float alpha = exp2f(m[h] - mn);
      const float pp = exp2f(zz - mn);
      ps[lane][h] = pp;
      l[h] = l[h] * alpha + group_sum<64>(pp);
#pragma unroll
      for (int c = 0; c < DPL; ++c) acc[h][c] *= alpha;
      m[h] = mn;
    }
    __syncthreads();
    for (int t = 0; t < ntok; ++t) {
      const T* vr = Vg + (size_t)(t0 + t) * D + lane * DPL;
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        const float v = to_f(vr[c]);
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][c] = fmaf(ps[t][h], v, acc[h][c]);
      }
    }
    __syncthreads();
    }
  }
  __shared__ float racc[G][D];
  __shared__ float rm[G], rl[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int c = 0; c < DPL; ++c) racc[h][lane * DPL + c] = acc[h][c];
    if (lane == 0) {
      rm[h] = m[h];
      rl[h] = l[h];
    }
  }
  __syncthreads();
  store_run<D, G, 64>(racc, rm, rl, slot_base(b, g, G, Hq, nsplit, split), nsplit, ws_acc,
                      ws_ml);
}

// ---------------------------------------------------------------- MFMA pass 1 (bf16)
template <int D, int G, int NW, int BS, bool FLAT>
__global__ __launch_bounds__(NW * 64) void attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, int K_max, float* __restrict__ ws_acc,
    float2* __restrict__ ws_ml, int Hq, int Hkv, int L, float qscale, int bps, int nsplit,
    int B, int nslot) {
  constexpr int KS = D / 32;   // MFMA k-steps over the head dim in q.K^T
  constexpr int NT = D / 16;   // 16-dim output tiles of P.V
  constexpr int DC = D / 8;    // lanes covering one V row (8 dims each) in the V loads
  constexpr int TG = 64 / DC;  // V rows per load instruction
  constexpr int TPL = DC;      // V loads per lane per chunk (= 64 / TG)
  constexpr int VP = D + 8;    // V tile row stride in LDS, in bf16 (16 B of padding)
  constexpr int TPB = BS / 16;                    // 16-token tiles per block
  constexpr int EPC = BS >= kChunk ? 1 : kChunk / BS;  // list entries per chunk
  constexpr int CPE = BS >= kChunk ? BS / kChunk : 1;  // chunks per list entry
  static_assert(G <= 8, "at most 8 query heads per KV head");
  static_assert(BS == 16 || BS == 32 || BS == 64 || BS == 128, "block of 16 to 128 tokens");
  static_assert(16 % TG == 0, "the rows of one V load lie in one tile");

  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, kg = lane >> 4;  // MFMA operand coordinates
  const int dc = lane % DC, tg = lane / DC;   // V load coordinates

  // With 8 waves there is no next-chunk K in flight: each wave loads K and V of its
  // chunk together (one chunk per wave in the plans that use 8 waves).
  constexpr bool PREFETCH = NW <= 4;
  static_assert(G * D * 4 <= kChunk * VP * 2, "a wave's O fits in its V tile");
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NW][kChunk * VP];
  __shared__ float mm[NW][G], ll[NW][G];
  // a wave's final O goes to its own V tile, which it no longer reads
  auto accs = [&](int w, int h, int dd) -> float& {
    return reinterpret_cast<float*>(Vs[w])[h * D + dd];
  };
  __shared__ float racc[G][D];
  __shared__ float rm[G], rl[G];

  // The B operand of S' = K.Q^T for query b: column = query head of the group (zero
  // beyond G), k = head dim.
  auto load_q = [&](int b, bf16x8_t (&qv)[KS]) {
    const bool hv = row < G;
    const uint16_t* qp = q + ((size_t)b * Hq + g * G + (hv ? row : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qp + s * 32 + kg * 8);
      if (!hv) v = bf16x8_t{};
      qv[s] = v;
    }
  };
  // The list entry this lane reads for a run of n_ent entries (wave-uniform count),
  // relative to the run's start, or -1 if it reads none. This wave's chunks are
  // wave + i*NW; their entries are read once, one per lane (at most 64 per wave; the
  // split plan keeps runs within that), so a chunk's tile starts are register reads,
  // not loads on the critical path.
  //   BS >= 64: lane i holds the entry of chunk i;
  //   BS <  64: lane i*EPC + u holds entry u of chunk i.
  auto entry_of_lane = [&](int n_ent) {
    const int n_chunks = BS >= kChunk ? n_ent * CPE : (n_ent + EPC - 1) / EPC;
    const int n_mine = (n_chunks - wave + NW - 1) / NW;
    const int i = lane / EPC, u = lane % EPC;
    const int e_rel = BS >= kChunk ? (wave + i * NW) / CPE : (wave + i * NW) * EPC + u;
    return i < n_mine && e_rel < n_ent ? e_rel : -1;
  };
  // Read ahead for a full list (count == K_max, the usual case when the cap binds): the
  // run of query blockIdx.z that this work-group then takes, and the query, are read
  // together with the counts instead of after them (one round trip instead of two
  // before the first K/V loads). A run that turns out different is read again.
  int run_spec = (K_max + nsplit - 1) / nsplit;
  run_spec = min((run_spec + EPC - 1) / EPC * EPC, bps);
  const int b_spec = blockIdx.z;
  const int j0_spec = blockIdx.x * run_spec;
  const int n_spec = max(0, min(j0_spec + run_spec, K_max) - j0_spec);
  int e_spec = -1;
  {
    const int r = entry_of_lane(n_spec);
    if (r >= 0) e_spec = sel_idx[(size_t)b_spec * K_max + j0_spec + r];
  }
  bf16x8_t q_spec[KS];
  load_q(b_spec, q_spec);

  // Entries [j0, j1) of query b's list (j0 < j1), reduced into slot `slot` of its heads;
  // `last`: no later slot of this query holds a partial.
  // (TrySpec false: the read-ahead is never used, so it need not stay live across a loop
  // of calls)
  auto run_entries = [&](int b, int j0, int j1, int slot, bool last, auto try_spec) {
    const bool spec =
        decltype(try_spec)::value && b == b_spec && j0 == j0_spec && j1 - j0 == n_spec;
    bf16x8_t qb[KS];
    if (spec) {
#pragma unroll
      for (int s = 0; s < KS; ++s) qb[s] = q_spec[s];
    } else {
      load_q(b, qb);
    }
    float m = -INFINITY, l = 0.f;  // online-softmax state of head `row`
    floatx4_t o[NT];               // o[dt][r] = O[head 4kg + r][dim 16dt + row]
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) o[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const int nbl = (L + BS - 1) / BS;
    const uint16_t* Kg = Kc + ((size_t)b * Hkv + g) * (size_t)L * D;
    const uint16_t* Vg = Vc + ((size_t)b * Hkv + g) * (size_t)L * D;
    const int n_ent = j1 - j0;
    const int n_chunks = BS >= kChunk ? n_ent * CPE : (n_ent + EPC - 1) / EPC;
    const int n_mine = (n_chunks - wave + NW - 1) / NW;
    int my_blk = -1;
    {
      int e = -1;
      if (spec) {
        e = e_spec;
      } else {
        const int r = entry_of_lane(n_ent);
        if (r >= 0) e = sel_idx[(size_t)b * K_max + j0 + r];
      }
      my_blk = (e < 0 || e >= nbl) ? -1 : e;  // entries outside [0, nbl) are ignored
    }
    // first token of each 16-token tile of chunk i, or -1 for a tile with no block
    auto tile_starts = [&](int i, int (&st)[4]) {
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        if constexpr (BS >= kChunk) {
          const int blk = __builtin_amdgcn_readlane(my_blk, i);
          const int off = ((wave + i * NW) % CPE) * kChunk + T * 16;
          st[T] = blk < 0 ? -1 : blk * BS + off;
        } else {
          const int blk = __builtin_amdgcn_readlane(my_blk, i * EPC + T / TPB);
          st[T] = blk < 0 ? -1 : blk * BS + (T % TPB) * 16;
        }
      }
    };
    // a chunk with no token below L is skipped (its scores would all be -inf)
    auto any_token = [&](const int (&st)[4]) {
      bool a = false;
#pragma unroll
      for (int T = 0; T < 4; ++T) a = a || (st[T] >= 0 && st[T] < L);
      return a;
    };
    // K rows of a chunk in the A-operand layout: lane (token row, k-group kg)
    auto load_k = [&](const int (&st)[4], bf16x8_t (&kb)[4][KS]) {
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        const int tok = st[T] < 0 ? 0 : min(st[T] + row, L - 1);
        const uint16_t* kp = Kg + (size_t)tok * D + kg * 8;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          kb[T][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(kp + s * 32));
      }
    };
    // V rows of a chunk: lane (dim chunk dc, row group tg), whole rows per instruction
    auto load_v = [&](const int (&st)[4], u32x4_t (&vv)[TPL]) {
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const int T = (i * TG) / 16;
        const int tok = st[T] < 0 ? 0 : min(st[T] + (i * TG) % 16 + tg, L - 1);
        vv[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(Vg + (size_t)tok * D + dc * 8));
      }
    };
    uint16_t* const vs = Vs[wave];
    // after_v runs once the chunk's V registers are stored to LDS (they may be reloaded
    // then), after_s once the score MFMAs have read the K registers
    // (a chunk with no token below L, active false, only stores V and runs the hooks:
    // the reloads then have one place in the code, which keeps the compiler from
    // hoisting them out of two branches above the uses of the registers they refill)
    auto consume = [&](const int (&st)[4], const bf16x8_t (&kb)[4][KS],
                       const u32x4_t (&vv)[TPL], bool active, auto&& after_v,
                       auto&& after_s) {
      // the chunk's V rows to this wave's LDS tile, row t = chunk token t
#pragma unroll
      for (int i = 0; i < TPL; ++i)
        *reinterpret_cast<u32x4_t*>(&vs[(i * TG + tg) * VP + dc * 8]) = vv[i];
      // the reloads stay where they are: hoisted above these uses they would need a
      // second register set
      __builtin_amdgcn_sched_barrier(0);
      after_v();
      // S'[token][head] for the 4 tiles: sc[T][r] = S'[chunk token 16T + 4kg + r][head row]
      floatx4_t sc[4];
      if (active) {
#pragma unroll
        for (int T = 0; T < 4; ++T) {
          floatx4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s)
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[T][s], qb[s], a, 0, 0, 0);
          sc[T] = a;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      after_s();
      if (!active) return;
      float bm = -INFINITY;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool tv = st[T] >= 0 && st[T] + 4 * kg + r < L;
          const float z = tv ? sc[T][r] * qscale : -INFINITY;
          sc[T][r] = z;
          bm = fmaxf(bm, z);
        }
      bm = xor32_max(xor16_max(bm));
      // the chunk has a token below L, so bm and mn are finite; alpha = 0 on the first chunk.
      // v_exp_f32 directly: arguments are <= 0 and results below 2^-126 weigh nothing.
      const float mn = fmaxf(m, bm);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      float rs = 0.f;
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(sc[T][r] - mn);
          sc[T][r] = p;
          rs += p;
        }
      rs = xor32_sum(xor16_sum(rs));
      l = l * alpha + rs;
      m = mn;
      // rescale O rows 4kg + r by their head's alpha, held by lane 4kg + r (rows >= G
      // are padding and take any finite factor)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float ar = readlane_f(alpha, r);
        if constexpr (G > 4) ar = kg == 1 ? readlane_f(alpha, 4 + r) : ar;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) o[dt][r] *= ar;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // O += P.V: A = P (k = tokens {32s+4kg..+3} then {32s+16+4kg..+3}, in bf16),
      // B = V from the transposing LDS read in the same token order
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8_t pa = {(__bf16)sc[2 * s][0],     (__bf16)sc[2 * s][1],
                             (__bf16)sc[2 * s][2],     (__bf16)sc[2 * s][3],
                             (__bf16)sc[2 * s + 1][0], (__bf16)sc[2 * s + 1][1],
                             (__bf16)sc[2 * s + 1][2], (__bf16)sc[2 * s + 1][3]};
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          // lane `row` receives V[32s + 4kg + k][16dt + row], k = 0..3, then the same 16
          // tokens later: the token order of pa
          const uint16_t* vp = &vs[(32 * s + 4 * kg + row / 4) * VP + dt * 16 + 4 * (row % 4)];
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, lds_tr_b_operand(vp, VP), o[dt],
                                                          0, 0, 0);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    if constexpr (PREFETCH) {
      // Software pipeline over this wave's chunks, one register set for K and one for
      // V: the next chunk's V is loaded into the V registers as soon as the current V
      // is in LDS, and its K into the K registers as soon as the score MFMAs have read
      // them, so both are in flight while the current chunk is consumed.
      int st[4] = {-1, -1, -1, -1};
      bf16x8_t kb[4][KS];
      u32x4_t vv[TPL];
      if (n_mine > 0) {
        tile_starts(0, st);
        load_v(st, vv);
        load_k(st, kb);
      }
      // (the last chunk has its own copy of the body: a conditional reload would keep
      // the old register values live beside the new ones)
      for (int i = 0; i + 1 < n_mine; ++i) {
        int stn[4];
        tile_starts(i + 1, stn);
        auto next_v = [&] { load_v(stn, vv); };
        auto next_k = [&] { load_k(stn, kb); };
        consume(st, kb, vv, any_token(st), next_v, next_k);
#pragma unroll
        for (int T = 0; T < 4; ++T) st[T] = stn[T];
      }
      if (n_mine > 0 && any_token(st)) consume(st, kb, vv, true, [] {}, [] {});
    } else {
      for (int i = 0; i < n_mine; ++i) {
        int st[4];
        tile_starts(i, st);
        bf16x8_t kb[4][KS];
        load_k(st, kb);
        u32x4_t vv[TPL];
        load_v(st, vv);
        if (any_token(st)) consume(st, kb, vv, true, [] {}, [] {});
      }
    }

    // this wave's state to LDS: heads h < G (O row h lives in lanes kg = h / 4, r = h % 4)
    if (lane < G) {
      mm[wave][lane] = m;
      ll[wave][lane] = l;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * kg + r;
      if (h < G) {
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) accs(wave, h, dt * 16 + row) = o[dt][r];
      }
    }
    __syncthreads();
    // merge the waves of this work-group into the run result
    for (int oi = threadIdx.x; oi < G * D; oi += NW * 64) {
      const int h = oi / D, dd = oi % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, mm[w][h]);
      float ls = 0.f, a = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = mm[w][h] == -INFINITY ? 0.f : exp2f(mm[w][h] - M);
        ls += sc * ll[w][h];
        a += sc * accs(w, h, dd);
      }
      racc[h][dd] = a;
      if (dd == 0) {
        rm[h] = M;
        rl[h] = ls;
      }
    }
    __syncthreads();
    store_run<D, G, NW * 64>(racc, rm, rl, slot_base(b, g, G, Hq, nslot, slot), nslot, ws_acc,
                             ws_ml, last);
  };

  if constexpr (FLAT) {
    // The B lists laid end to end in query order and cut into runs of one length
    // `chunk`, ceil(total / (nsplit * B)) entries: work-group x + nsplit*z takes run
    // number x + nsplit*z, so queries that select very different numbers of blocks keep
    // the work-groups equally busy. A run may end one query's list and start the next
    // one's: it reduces each part into a partial of that query, in the query's slot
    // (run number - first run touching the query), and the run holding a query's last
    // entry marks that partial as the last. chunk >= ceil(max count / (nslot - 1)) keeps
    // every query within its nslot slots. With nearly equal counts (nsplit runs per
    // query no longer than chunk) the per-query runs are kept: every work-group then
    // reduces one query's run, with no run split between two queries. Every wave reduces
    // the B counts itself (no barrier): lane b holds query b's count.
    const int c = lane < B ? min(max(sel_cnt[lane], 0), K_max) : 0;
    const int wg = nsplit * B;
    const int end_incl = (int)wave_incl_scan((uint32_t)c);  // lane b: end of b's list
    const int total = __builtin_amdgcn_readlane(end_incl, 63);
    const float maxf = wave_max_to_last((float)c);  // counts are exact in fp32
    const int maxc = (int)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(maxf), 63));
    const int lo = (maxc + nslot - 2) / (nslot - 1);  // nslot >= 2 in flat plans
    int chunk = max(max(lo, 1), (total + wg - 1) / wg);
    chunk = (chunk + EPC - 1) / EPC * EPC;
    int per_query = (maxc + nsplit - 1) / nsplit;
    per_query = (per_query + EPC - 1) / EPC * EPC;
    if (per_query <= chunk || chunk > bps) {
      const int split = blockIdx.x, b = blockIdx.z;
      const int cnt = __builtin_amdgcn_readlane(c, b);
      int run = (cnt + nsplit - 1) / nsplit;
      run = min((run + EPC - 1) / EPC * EPC, bps);
      const int j0 = split * run;
      const bool last = split == nsplit - 1;  // every slot is written; the last is marked
      const size_t base = slot_base(b, g, G, Hq, nslot, split);
      if (j0 < cnt)
        run_entries(b, j0, min(j0 + run, cnt), split, last, std::true_type{});
      else if (last)
        store_end_marker<G>(base, nslot, ws_ml);
      else
        store_empty_run<G>(base, nslot, ws_ml);
    } else {
      const int sidx = blockIdx.x + nsplit * blockIdx.z;
      if (sidx == 0) {  // queries with no entry: an empty last partial in their first slot
        for (int b = 0; b < B; ++b)
          if (__builtin_amdgcn_readlane(c, b) == 0)
            store_end_marker<G>(slot_base(b, g, G, Hq, nslot, 0), nslot, ws_ml);
      }
      const int s0 = sidx * chunk, s1 = min(s0 + chunk, total);
      // the queries with entries in [s0, s1), lowest first (a wave-uniform mask, the same
      // in every wave of the work-group)
      uint64_t touch = __ballot(c > 0 && end_incl > s0 && end_incl - c < s1);
      while (touch) {
        const int b = __builtin_ctzll(touch);
        touch &= touch - 1;
        const int e = __builtin_amdgcn_readlane(end_incl, b);
        const int beg = e - __builtin_amdgcn_readlane(c, b);
        run_entries(b, max(s0, beg) - beg, min(s1, e) - beg, sidx - beg / chunk, e <= s1,
                    std::false_type{});
      }
    }
  } else {
    const int split = blockIdx.x, b = blockIdx.z;
    const int cnt = min(max(sel_cnt[b], 0), K_max);
    // Runs are cut from this row's actual count, spread over all nsplit work-groups
    // (whole chunks for small blocks); `bps` is the split plan's maximum, sized for
    // K_max, and cnt <= K_max keeps every run within it.
    int run = (cnt + nsplit - 1) / nsplit;
    run = min((run + EPC - 1) / EPC * EPC, bps);
    const int j0 = split * run;
    if (j0 >= cnt)
      store_empty_run<G>(slot_base(b, g, G, Hq, nslot, split), nslot, ws_ml);
    else
      run_entries(b, j0, min(j0 + run, cnt), split, false, std::true_type{});
  }
}

// ---------------------------------------------------------------- merge of the runs
// Above 32 slots: one work-group per (query, head); thread = head dim. The head's slots
// are read CH at a time (16, or 8 when runs are marked) -- one memory round trip per CH
// slots -- and merged with an online rescale in slot order, up to nslot slots or
// (MARKED) the partial marked last, whichever comes first; empty runs carry m = -inf.
// A row with no selected token (every m = -inf) gets zeros. (Reading 32 slots per
// round trip this way, 64 loads in flight per thread, was 2 us slower per 128K batch-8
// call than 8 at a time.)
template <typename T, int D, bool MARKED, int CH>
__global__ __launch_bounds__(D) void attn_combine(const float* __restrict__ ws_acc,
                                                  const float2* __restrict__ ws_ml,
                                                  T* __restrict__ out, int nslot) {
  const int rowi = blockIdx.x;  // b * Hq + hq
  const float2* ml = ws_ml + (size_t)rowi * nslot;
  const float* ap = ws_acc + (size_t)rowi * nslot * D + threadIdx.x;
  float M = -INFINITY, ls = 0.f, a = 0.f;
  for (int s0 = 0; s0 < nslot; s0 += CH) {
    float2 v[CH];
    float x[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool ok = s0 + i < nslot;
      // both loads issue together; an empty run's acc slot may hold anything
      v[i] = ok ? ml[s0 + i] : make_float2(-INFINITY, 0.f);
      x[i] = ok ? ap[(size_t)(s0 + i) * D] : 0.f;
    }
    // the last partial (l < 0, stored as -l - 1) ends the slots; any after it are stale
    bool end = false;
    if constexpr (MARKED) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (end) v[i].x = -INFINITY;
        if (!end && v[i].y < 0.f) {
          v[i].y = -v[i].y - 1.f;
          end = true;
        }
      }
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < CH; ++i) Mc = fmaxf(Mc, v[i].x);
    if (Mc != -INFINITY) {
      const float sc = M == -INFINITY ? 0.f : exp2f(M - Mc);
      ls *= sc;
      a *= sc;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (v[i].x != -INFINITY) {
          const float w = exp2f(v[i].x - Mc);
          ls += w * v[i].y;
          a += w * x[i];
        }
      }
      M = Mc;
    }
    if (MARKED && end) break;
  }
  store_out(out + (size_t)rowi * D + threadIdx.x, ls > 0.f ? a / ls : 0.f);
}

// The merge for at most 32 slots, every load in one round trip: 256 threads, each
// holding 16-byte pieces of the head's slots (slot t / (D/4) + k * 1024 / D, dims
// 4 (t % (D/4)) .. +3), and in every wave lane s holding slot s's (m, l). Each wave finds
// the marked slot (MARKED), the maximum M and the weights w_s = 2^(m_s - M) itself, so
// the only barrier is the one of the final sum over the threads that share a piece of
// the head dims (lane swaps inside a wave, then LDS across the four waves). Slots past
// the marked one, and the acc of empty runs, are never read into the sums. Against the
// per-dim merge above with 8 slots per round trip: 128K batch 1 call 17.8 -> 15.8 us,
// page geometry 27.4 -> 25.3, batch 8 with spread budgets 43.8 -> 43.0, batch 8 equal
// budgets unchanged (84.3-84.5).
template <typename T, int D, bool MARKED>
__global__ __launch_bounds__(256) void attn_merge32(const float* __restrict__ ws_acc,
                                                    const float2* __restrict__ ws_ml,
                                                    T* __restrict__ out, int nslot) {
  constexpr int NV = D / 4;            // 16-byte pieces per slot: 32 (d 128) or 16 (d 64)
  constexpr int PER = 32 * NV / 256;   // pieces per thread
  constexpr int SPT = 256 / NV;        // slot step between a thread's pieces
  const int rowi = blockIdx.x;  // b * Hq + hq
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float4* ap = reinterpret_cast<const float4*>(ws_acc + (size_t)rowi * nslot * D);
  // slots 0 .. SPT-1 (the first piece of every thread) are read with the (m, l) pairs;
  // the rest with them too when every slot holds a run, else only up to the marked slot
  // once it is known (a second round trip only for heads with more than SPT runs)
  float4 x[PER];
  x[0] = t / NV < nslot ? ap[t] : make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (!MARKED) {
#pragma unroll
    for (int k = 1; k < PER; ++k)
      x[k] = t / NV + SPT * k < nslot ? ap[t + 256 * k] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float2 ml = lane < nslot ? ws_ml[(size_t)rowi * nslot + lane] : make_float2(-INFINITY, 0.f);
  bool valid = lane < nslot;
  if constexpr (MARKED) {
    // the first marked slot (l stored as -l - 1) is the last one of this head
    const uint64_t mk = __ballot(valid && ml.y < 0.f);
    int e = nslot - 1;
    if (mk != 0) {
      e = __builtin_ctzll(mk);
      valid = valid && lane <= e;
      if (lane == e) ml.y = -ml.y - 1.f;
    }
#pragma unroll
    for (int k = 1; k < PER; ++k)
      x[k] = t / NV + SPT * k <= e ? ap[t + 256 * k] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float m = valid ? ml.x : -INFINITY;
  const float M = readlane_f(wave_max_to_last(m), 63);
  const float w = m == -INFINITY ? 0.f : exp2f(m - M);  // M = -inf: every w is 0
  const float L = group_sum_dpp<64>(w > 0.f ? w * ml.y : 0.f);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float wk = __shfl(w, t / NV + SPT * k);
    if (wk > 0.f) {
      a.x += wk * x[k].x;
      a.y += wk * x[k].y;
      a.z += wk * x[k].z;
      a.w += wk * x[k].w;
    }
  }
  // threads t and t + NV (, t + 2 NV, t + 3 NV) of a wave hold the same dims
  auto wsum = [](float v) {
    if constexpr (NV == 16) v = xor16_sum(v);
    return xor32_sum(v);
  };
  a = make_float4(wsum(a.x), wsum(a.y), wsum(a.z), wsum(a.w));
  __shared__ float4 red[4][NV];
  if (lane < NV) red[wave][lane] = a;
  __syncthreads();
  if (t < NV) {
    float4 r = red[0][t];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      r.x += red[i][t].x;
      r.y += red[i][t].y;
      r.z += red[i][t].z;
      r.w += red[i][t].w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T* o = out + (size_t)rowi * D + 4 * t;
    store_out(o + 0, r.x * inv);
    store_out(o + 1, r.y * inv);
    store_out(o + 2, r.z * inv);
    store_out(o + 3, r.w * inv);
  }
}

struct Ws {
  float* acc;
  float2* ml;
};

Ws carve(void* workspace, int B, int Hq, int d, int nslot) {
  Ws w;
  w.acc = static_cast<float*>(workspace);
  w.ml = reinterpret_cast<float2*>(w.acc + (size_t)B * Hq * nslot * d);
  return w;
}

template <typename T, int D, int G>
hipError_t launch_generic(const void* q, const void* k, const void* v, const int32_t* sel_idx,
                          const int32_t* sel_cnt, int K_max, Ws ws, void* out, int B, int Hq,
                          int Hkv, int L, int block, float qscale, AttnSplit sp,
                          hipStream_t stream) {
  dim3 grid(sp.nsplit, Hkv, B);
  hipLaunchKernelGGL((attn_generic<T, D, G>), grid, dim3(64), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), sel_idx, sel_cnt, K_max, ws.acc, ws.ml, Hq, Hkv,
                     L, qscale, block, sp.blocks_per_split, sp.nsplit);
  return hipGetLastError();
}

template <int D, int G, int BS>
hipError_t launch_mfma_bs(const void* q, const void* k, const void* v, const int32_t* sel_idx,
                          const int32_t* sel_cnt, int K_max, Ws ws, int B, int Hq, int Hkv,
                          int L, float qscale, AttnSplit sp, hipStream_t stream) {
  // the kernel keeps a wave's list entries one per lane: at most 64 of them
  const int entries_per_chunk = BS >= kChunk ? 1 : kChunk / BS;
  const long chunks = BS >= kChunk ? (long)sp.blocks_per_split * (BS / kChunk)
                                   : (sp.blocks_per_split + entries_per_chunk - 1) /
                                         entries_per_chunk;
  if ((chunks + sp.waves - 1) / sp.waves * entries_per_chunk > 64)
    return hipErrorNotSupported;  // a plan this kernel cannot hold (the plan never makes one)
#define SPOT_MFMA(NW, FLAT, GRID)                                                             \
  hipLaunchKernelGGL((attn_mfma<D, G, NW, BS, FLAT>), GRID, dim3(NW * 64), 0, stream,         \
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),        \
                     static_cast<const uint16_t*>(v), sel_idx, sel_cnt, K_max, ws.acc, ws.ml, \
                     Hq, Hkv, L, qscale, sp.blocks_per_split, sp.nsplit, B, sp.nslot)
  const dim3 grid(sp.nsplit, Hkv, B);
  if (sp.waves == 8) {
    if (sp.flat)
      SPOT_MFMA(8, true, grid);
    else
      SPOT_MFMA(8, false, grid);
  } else if (sp.flat) {
    SPOT_MFMA(4, true, grid);
  } else {
    SPOT_MFMA(4, false, grid);
  }
#undef SPOT_MFMA
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_mfma(const void* q, const void* k, const void* v, const int32_t* sel_idx,
                       const int32_t* sel_cnt, int K_max, Ws ws, void* out, int B, int Hq,
                       int Hkv, int L, int block, float qscale, AttnSplit sp,
                       hipStream_t stream) {
  switch (block) {
    case 16:
      return launch_mfma_bs<D, G, 16>(q, k, v, sel_idx, sel_cnt, K_max, ws, B, Hq, Hkv, L,
                                      qscale, sp, stream);
    case 32:
      return launch_mfma_bs<D, G, 32>(q, k, v, sel_idx, sel_cnt, K_max, ws, B, Hq, Hkv, L,
                                      qscale, sp, stream);
    case 128:
      return launch_mfma_bs<D, G, 128>(q, k, v, sel_idx, sel_cnt, K_max, ws, B, Hq, Hkv, L,
                                       qscale, sp, stream);
    default:
      return launch_mfma_bs<D, G, 64>(q, k, v, sel_idx, sel_cnt, K_max, ws, B, Hq, Hkv, L,
                                      qscale, sp, stream);
  }
}

template <typename T, int D>
hipError_t launch_d(const void* q, const void* k, const void* v, bool fast,
                    const int32_t* sel_idx, const int32_t* sel_cnt, int K_max, Ws ws,
                    void* out, int B, int Hq, int Hkv, int L, int block, float qscale,
                    AttnSplit sp, hipStream_t stream) {
  const int G = Hq / Hkv;
  hipError_t e;
#define SPOT_ARGS \
  q, k, v, sel_idx, sel_cnt, K_max, ws, out, B, Hq, Hkv, L, block, qscale, sp, stream
  if (std::is_same<T, uint16_t>::value && fast) {
    switch (G) {
      case 1: e = launch_mfma<D, 1>(SPOT_ARGS); break;
      case 2: e = launch_mfma<D, 2>(SPOT_ARGS); break;
      case 4: e = launch_mfma<D, 4>(SPOT_ARGS); break;
      default: e = launch_mfma<D, 8>(SPOT_ARGS); break;
    }
  } else {
    switch (G) {
      case 1: e = launch_generic<T, D, 1>(SPOT_ARGS); break;
      case 2: e = launch_generic<T, D, 2>(SPOT_ARGS); break;
      case 4: e = launch_generic<T, D, 4>(SPOT_ARGS); break;
      default: e = launch_generic<T, D, 8>(SPOT_ARGS); break;
    }
  }
#undef SPOT_ARGS
  if (e != hipSuccess) return e;
  // The merge: runs cut across the batch (flat plans) flag each query's last partial,
  // so their merge stops there; runs per query fill all nsplit slots. Up to 32 slots
  // per head the one-round-trip merge, above that the slot-by-slot one.
  if (sp.nslot <= 32 && sp.flat)
    hipLaunchKernelGGL((attn_merge32<T, D, true>), dim3(B * Hq), dim3(256), 0, stream, ws.acc,
                       ws.ml, static_cast<T*>(out), sp.nslot);
  else if (sp.nslot <= 32)
    hipLaunchKernelGGL((attn_merge32<T, D, false>), dim3(B * Hq), dim3(256), 0, stream, ws.acc,
                       ws.ml, static_cast<T*>(out), sp.nslot);
  else if (sp.flat)
    hipLaunchKernelGGL((attn_combine<T, D, true, 8>), dim3(B * Hq), dim3(D), 0, stream, ws.acc,
                       ws.ml, static_cast<T*>(out), sp.nslot);
  else
    hipLaunchKernelGGL((attn_combine<T, D, false, 16>), dim3(B * Hq), dim3(D), 0, stream,
                       ws.acc, ws.ml, static_cast<T*>(out), sp.nslot);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                              bool bf16, const int32_t* sel_idx, const int32_t* sel_cnt,
                              int K_max, void* out, void* workspace, int B, int Hq, int Hkv,
                              int d, int L, int block, float sm_scale, hipStream_t stream) {
  const bool fast = bf16;
  const AttnSplit sp = attn_split_plan(B, Hkv, K_max, block, fast);
  const Ws ws = carve(workspace, B, Hq, d, sp.nslot);
  const float qscale = sm_scale * kLog2e;
  if (bf16)
    return d == 64 ? launch_d<uint16_t, 64>(q, k_cache, v_cache, fast, sel_idx, sel_cnt, K_max,
                                            ws, out, B, Hq, Hkv, L, block, qscale, sp, stream)
                   : launch_d<uint16_t, 128>(q, k_cache, v_cache, fast, sel_idx, sel_cnt, K_max,
                                             ws, out, B, Hq, Hkv, L, block, qscale, sp, stream);
  return d == 64 ? launch_d<float, 64>(q, k_cache, v_cache, false, sel_idx, sel_cnt, K_max, ws,
                                       out, B, Hq, Hkv, L, block, qscale, sp, stream)
                 : launch_d<float, 128>(q, k_cache, v_cache, false, sel_idx, sel_cnt, K_max, ws,
                                        out, B, Hq, Hkv, L, block, qscale, sp, stream);
}

// ---------------------------------------------------------------- allocation-free form
// The workspace of spot_sparse_attn_noalloc: a file-scope device array (each GPU holds its
// own copy from the moment the library's code is loaded on it until the process ends).
// In host code `scratch` names a host-side stand-in, not a device address: the device
// address of a GPU's copy comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(scratch_once[dev], [dev] {
    // the lookup runs with the stream's device current, then the caller's is restored
    int cur = -1;
    scratch_err[dev] = hipGetDevice(&cur);
    if (scratch_err[dev] == hipSuccess && cur != dev) scratch_err[dev] = hipSetDevice(dev);
    if (scratch_err[dev] == hipSuccess) {
      void* p = nullptr;
      scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      scratch_ptr[dev] = p;
    }
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (scratch_err[dev] == hipSuccess) scratch_err[dev] = r;
    }
  });
  *ptr = scratch_ptr[dev];
  return scratch_err[dev];
}

}  // namespace spot
