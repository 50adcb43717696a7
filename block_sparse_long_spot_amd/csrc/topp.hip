// Dual top-p block selection (SpotAttention §2.3, Eq. 7 and Eq. 8).
//
// One work-group per query row; latency-bound (a few thousand scores), so the design
// minimises the chain of dependent steps: 6 work-group barriers (7 when the boundary
// bin below holds more than 8 blocks), wave-level scans on
// the DPP network, one 64-bit LDS atomic per block. Every thread keeps EPT consecutive
// blocks in registers: the score, an order-preserving 32-bit key of it, and the
// block's softmax mass exp(s - max) in 2^-29 fixed point (integer sums are exact, so
// nothing depends on the order in which threads add).
//
//   1. reserved blocks R (sink prefix, recency suffix) are set aside;
//   2. max over the residual blocks, then each residual block's mass (Eq. 7);
//   3. one coarse histogram over 2048 bins of width 1/64 in (max - s) (bin order =
//      score order) holding (count << 44) | mass per bin, and its prefix sums. One pass
//      over the prefix finds the bin where the cumulative mass reaches p*Z (the nucleus
//      cut) and the bins of the two block counts the clamp
//      k = clamp(k_p, K_min - r, K_max - r) can produce; as the clamp is monotone this
//      decides whether k is already known or falls inside the cut bin;
//   4. only the bin holding the k-th block needs an exact order: its blocks (usually a
//      handful) are gathered and ranked by (score desc, index asc), by every wave for
//      a handful, split over the waves for more, accumulating mass in that order to
//      finish k_p when needed. A bin with more than
//      64 blocks (dense ties) falls back to an exact radix select, 11+11+10 bits of
//      the key, restricted to that bin;
//   5. blocks in earlier bins, the chosen ones of the boundary bin, and R form S; a
//      block-wide scan writes it in ascending order.
#include "device_common.h"
#include "spot_internal.h"

namespace spot {
namespace {

typedef unsigned long long u64;

constexpr int kCoarseBins = 2048;
constexpr float kBinsPerNat = 64.f;  // coarse bin width: 1/64 of a unit of log-mass
constexpr int kRankMax = 64;         // boundary bins up to this size are ranked by one wave
constexpr int kRankRedundant = 8;    // up to this size every wave ranks the whole bin
constexpr int kMassBits = 29;        // fixed point of a block's mass (<= 1.0)
constexpr int kCntShift = 44;        // count field of a packed bin: 16384 blocks * 2^29 < 2^44
constexpr u64 kMassMask = (1ull << kCntShift) - 1;

template <int NT>
struct ToppSmem {
  u64 hist[kCoarseBins];             // packed coarse histogram (count << 44) | mass
  uint32_t hc[kCoarseBins];          // fallback radix histograms
  u64 hm[kCoarseBins];
  uint32_t gk[kRankMax];             // gathered boundary-bin blocks: key, index, mass
  int32_t gi[kRankMax];
  u64 gm[kRankMax];
  uint32_t grank[kRankMax];          // their rank and the mass ranked before them, summed
  u64 gcm[kRankMax];                 // over the waves (bins of more than kRankRedundant)
  int32_t ng;
  // bins found by the prefix pass: [0] mass target, [1] low count target, [2] high
  int32_t f_bin[3];
  u64 f_pre[3];                      // packed prefix (blocks and mass above the bin)
  u64 f_cnt[3];                      // blocks in the bin
  u64 wt[NT / 64];                   // per-wave totals
  u64 wt2[NT / 64];
  float wf[NT / 64];
  uint32_t r_digit;
  u64 r_cnt_above;
  u64 r_mass_above;
};

// Sum over the work-group (one barrier; `slot` must not be in use).
template <int NT>
__device__ u64 block_sum(u64 v, u64* slot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const u64 w = lane_value(wave_incl_scan(v), 63);
  if (lane == 0) slot[wave] = w;
  __syncthreads();
  u64 r = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r += slot[i];
  return r;
}

// Exclusive prefix sum in thread order, and the total (one barrier).
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, u64* slot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) slot[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = static_cast<uint32_t>(slot[w]);
    before += w < wave ? t : 0u;
    tot += t;
  }
  total = tot;
  return before + x - v;
}

// Radix select over the active keys, from the largest key down (fallback path).
// BY_MASS: stop where the cumulative mass reaches `target`; otherwise where the
// cumulative count does. Outputs the selected key, the count and mass strictly above
// it, and the count and mass of its tie group.
template <int NT, int EPT, bool BY_MASS>
__device__ void radix_select(const uint32_t (&key)[EPT], const u64 (&mass)[EPT],
                             const bool (&act)[EPT], u64 target, ToppSmem<NT>& sh,
                             uint32_t& tau, u64& cnt_above, u64& mass_above, u64& tie_cnt,
                             u64& tie_mass) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, pmask = 0;
  cnt_above = 0;
  mass_above = 0;
  uint32_t digit = 0;
  if (tid == 0) {  // a crossing is always found; this only keeps the slot defined
    sh.r_digit = 0;
    sh.r_cnt_above = 0;
    sh.r_mass_above = 0;
  }
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    const uint32_t dmask = nbins - 1;
    for (int i = tid; i < nbins; i += NT) {
      sh.hc[i] = 0;
      sh.hm[i] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (act[e] && (key[e] & pmask) == prefix) {
        const uint32_t d = (key[e] >> shift) & dmask;
        atomicAdd(&sh.hc[d], 1u);
        if (BY_MASS) atomicAdd(&sh.hm[d], mass[e]);
      }
    }
    __syncthreads();
    // thread t owns bins [t*bpt, t*bpt + bpt); scan them from the top
    const int bpt = nbins / NT;
    const int b0 = tid * bpt;
    u64 lc = 0, lm = 0;
    for (int i = 0; i < bpt; ++i) {
      lc += sh.hc[b0 + i];
      if (BY_MASS) lm += sh.hm[b0 + i];
    }
    // inclusive suffix sums across lanes (lane i: sum over lanes >= i)
    u64 sc = lc, sm = lm;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const u64 yc = __shfl_down(sc, o, 64);
      const u64 ym = __shfl_down(sm, o, 64);
      if (lane + o < 64) {
        sc += yc;
        sm += ym;
      }
    }
    if (lane == 0) {
      sh.wt[wave] = sc;
      sh.wt2[wave] = sm;
    }
    __syncthreads();
    u64 hc_hi = 0, hm_hi = 0;  // totals of the waves holding higher bins
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      if (w > wave) {
        hc_hi += sh.wt[w];
        hm_hi += sh.wt2[w];
      }
    }
    const u64 ec = sc - lc + hc_hi;  // count in bins above this thread's bins
    const u64 em = sm - lm + hm_hi;
    const u64 need = BY_MASS ? target - mass_above : target - cnt_above;
    const u64 ex = BY_MASS ? em : ec;
    const u64 lx = BY_MASS ? lm : lc;
    if (ex < need && ex + lx >= need) {
      u64 rc = ec, rm = em;
      for (int i = bpt - 1; i >= 0; --i) {
        const u64 c = sh.hc[b0 + i];
        const u64 m = BY_MASS ? sh.hm[b0 + i] : 0;
        if ((BY_MASS ? rm + m : rc + c) >= need) {
          sh.r_digit = b0 + i;
          sh.r_cnt_above = rc;
          sh.r_mass_above = rm;
          break;
        }
        rc += c;
        rm += m;
      }
    }
    __syncthreads();
    digit = sh.r_digit & dmask;
    cnt_above += sh.r_cnt_above;
    mass_above += sh.r_mass_above;
    prefix |= digit << shift;
    pmask |= dmask << shift;
  }
  tau = prefix;
  tie_cnt = sh.hc[digit];
  tie_mass = sh.hm[digit];
  __syncthreads();
}

// exp(s - mx) in 2^-29 fixed point. s - mx and its split into an integer and a
// fraction are exact in fp64; only the fractional power of two is evaluated in fp32, by
// the hardware exponential on [0, 1) (about 1 ulp), so the mass carries a relative error
// near 1e-7. The result is at most 2^29.
__device__ __forceinline__ u64 fixed_mass(float s, float mx) {
  const double t = (static_cast<double>(s) - static_cast<double>(mx)) * 1.4426950408889634;
  const double n = floor(t);
  if (n < -60.0) return 0ull;
  const float f = static_cast<float>(t - n);                            // in [0, 1)
  const float v = ldexpf(__builtin_amdgcn_exp2f(f), static_cast<int>(n) + kMassBits);
  return static_cast<u64>(static_cast<uint32_t>(__builtin_rintf(v)));
}

// Rows of prefill tiles (n_tiles > 0): row b is tile b % n_tiles of a sequence of T
// queries cut into tiles of Tq starting at position q_pos0; it sees the first
// ceil((q_pos0 + last query of the tile + 1) / block) blocks of its score row, so its
// recency window ends at the tile's diagonal. n_tiles == 0: every row has nb blocks.
struct RowGeom {
  int n_tiles, T, Tq, q_pos0, block;
};

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void select_topp_kernel(const float* __restrict__ scores,
                                                         int32_t* __restrict__ sel_idx,
                                                         int32_t* __restrict__ sel_cnt,
                                                         float* __restrict__ sel_mass,
                                                         int nb_stride, float p, int K_min,
                                                         int K_max, int n_sink, int n_rec,
                                                         RowGeom geom) {
  constexpr int BPT = kCoarseBins / NT;
  constexpr int NW = NT / 64;
  __shared__ ToppSmem<NT> sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = scores + (size_t)b * nb_stride;
  int nb = nb_stride;  // blocks of this row
  if (geom.n_tiles > 0) {
    const int q_end = min((b % geom.n_tiles + 1) * geom.Tq, geom.T);  // past the tile
    nb = min(nb_stride, (geom.q_pos0 + q_end + geom.block - 1) / geom.block);
  }
  const int rs = min(n_sink, nb), rr = min(n_rec, nb);
  const int r = min(nb, rs + rr);
  const int n_res = nb - r;
  const int lo = max(0, K_min - r);
  const int hi_cap = min(K_max - r, n_res);  // K_max >= r is checked on the host
  // k as a function of the nucleus size: monotone in k_p
  auto clampk = [&](int x) { return min(max(x, lo), hi_cap); };

  // ---- 1. scores into registers; clear the histogram
  float s[EPT];
  uint32_t key[EPT];
  bool valid[EPT], res[EPT];
  if ((nb_stride & 3) == 0 && (EPT & 3) == 0) {
    // whole float4s of the row (nb_stride % 4 == 0 keeps them inside it)
#pragma unroll
    for (int e = 0; e < EPT; e += 4) {
      const int i = tid * EPT + e;
      const float4 v4 = i < nb ? *reinterpret_cast<const float4*>(row + i)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      s[e] = v4.x;
      s[e + 1] = v4.y;
      s[e + 2] = v4.z;
      s[e + 3] = v4.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int i = tid * EPT + e;
      s[e] = i < nb ? row[i] : 0.f;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid * EPT + e;
    valid[e] = i < nb;
    if (s[e] == 0.f) s[e] = 0.f;  // fold -0.0 onto +0.0
    key[e] = float_key(s[e]);
    res[e] = valid[e] && i >= rs && i < nb - rr;
    if (res[e]) mx = fmaxf(mx, s[e]);
  }
#pragma unroll
  for (int i = 0; i < BPT; ++i) sh.hist[tid * BPT + i] = 0;
  if (tid < kRankMax) {
    sh.grank[tid] = 0;
    sh.gcm[tid] = 0;
  }
  if (tid == 0) {
    sh.ng = 0;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      sh.f_bin[t] = 0;
      sh.f_pre[t] = 0;
      sh.f_cnt[t] = 0;
    }
  }
  // ---- 2. residual max, masses, coarse bins, histogram
  mx = wave_max_to_last(mx);
  if (lane == 63) sh.wf[wave] = mx;
  __syncthreads();  // barrier 1
  mx = sh.wf[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, sh.wf[w]);
  u64 mass[EPT];
  int cb[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    mass[e] = 0;
    cb[e] = -1;
    if (res[e]) {
      mass[e] = fixed_mass(s[e], mx);
      cb[e] = static_cast<int>(fminf((mx - s[e]) * kBinsPerNat, kCoarseBins - 1.f));
      atomicAdd(&sh.hist[cb[e]], (1ull << kCntShift) | mass[e]);
    }
  }
  __syncthreads();  // barrier 2
  // ---- 3. prefix over the bins (ascending bin = descending score)
  u64 hb[BPT];
  u64 loc = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    hb[i] = sh.hist[tid * BPT + i];
    loc += hb[i];
  }
  const u64 incl = wave_incl_scan(loc);
  if (lane == 63) sh.wt[wave] = incl;
  __syncthreads();  // barrier 3
  u64 before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const u64 t = sh.wt[w];
    before += w < wave ? t : 0ull;
    total += t;
  }
  const u64 Z = total & kMassMask;
  u64 T = 0;  // mass target of the nucleus cut
  int tl = 0, th = 0;
  int k = 0;
  if (n_res > 0) {
    if (p >= 1.f || p <= 0.f) {
      k = clampk(p >= 1.f ? n_res : 0);
      tl = k;
    } else {
      T = static_cast<u64>(ceil(static_cast<double>(p) * static_cast<double>(Z)));
      if (T == 0) T = 1;
      tl = min(max(lo, 1), hi_cap);
      th = hi_cap;
    }
  }
  {
    // Target t (0: mass T, 1: count tl, 2: count th) is reached in the one bin whose
    // prefix is below it and whose prefix plus content is not. The threads' bin ranges
    // partition the prefix, so one thread holds that bin: it is the thread whose whole
    // range brackets the target (one test per thread), and only it looks at its bins.
    const u64 P0 = before + incl - loc;  // packed prefix above this thread's bins
    const u64 P1 = before + incl;        // ... and above the bins after them
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const u64 X = t == 0 ? T : static_cast<u64>(t == 1 ? tl : th);
      if (X == 0) continue;  // uniform
      const u64 lo_x = t == 0 ? (P0 & kMassMask) : (P0 >> kCntShift);
      const u64 hi_x = t == 0 ? (P1 & kMassMask) : (P1 >> kCntShift);
      if (lo_x < X && X <= hi_x) {
        u64 P = P0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
          const u64 below = t == 0 ? (P & kMassMask) : (P >> kCntShift);
          const u64 in = t == 0 ? (hb[i] & kMassMask) : (hb[i] >> kCntShift);
          if (below < X && X <= below + in) {
            sh.f_bin[t] = tid * BPT + i;
            sh.f_pre[t] = P;
            sh.f_cnt[t] = hb[i] >> kCntShift;
          }
          P += hb[i];
        }
      }
    }
  }
  __syncthreads();  // barrier 4
  // ---- decide k, or the bin where it is decided
  // the three found bins, read together
  int fbin[3];
  u64 fpre[3], fcnt[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    fbin[t] = sh.f_bin[t];
    fpre[t] = sh.f_pre[t];
    fcnt[t] = sh.f_cnt[t];
  }
  int bk = -1;           // bin holding the k-th residual block in score order
  int fs = 0;            // which found slot describes bin bk
  bool need_kp = false;  // k still depends on the exact nucleus size inside bin bk
  if (n_res > 0) {
    if (T == 0) {
      if (k > 0) {
        bk = fbin[1];
        fs = 1;
      }
    } else {
      const int A0 = static_cast<int>(fpre[0] >> kCntShift);
      const int C0 = static_cast<int>(fcnt[0]);
      const int k1 = clampk(A0 + 1), k2 = clampk(A0 + C0);
      if (k1 != k2) {
        bk = fbin[0];
        need_kp = true;
      } else {
        k = k1;
        fs = k == th ? 2 : (k == tl ? 1 : 0);
        if (k > 0) bk = fs == 2 ? fbin[2] : (fs == 1 ? fbin[1] : fbin[0]);
      }
    }
  }
  const u64 fpre_s = fs == 2 ? fpre[2] : (fs == 1 ? fpre[1] : fpre[0]);
  const u64 fcnt_s = fs == 2 ? fcnt[2] : (fs == 1 ? fcnt[1] : fcnt[0]);
  const int A = bk >= 0 ? static_cast<int>(fpre_s >> kCntShift) : 0;
  const int C = bk >= 0 ? static_cast<int>(fcnt_s) : 0;
  const u64 PM = bk >= 0 ? (fpre_s & kMassMask) : 0;

  // ---- 4. exact order inside the boundary bin
  uint32_t tau = 0;
  u64 take = 0;  // fallback: blocks of key tau to take, lowest index first
  int slot[EPT];
  bool fallback = false;
  u64 chosen_mask = 0;  // gathered boundary-bin blocks that are chosen (bit = slot)
  u64 inbin_mass = 0;   // their mass
#pragma unroll
  for (int e = 0; e < EPT; ++e) slot[e] = 0;
  if (bk >= 0) {
    if (C <= kRankMax) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        if (cb[e] == bk) {
          const int sl = atomicAdd(&sh.ng, 1);
          slot[e] = sl;
          sh.gk[sl] = key[e];
          sh.gi[sl] = tid * EPT + e;
          sh.gm[sl] = mass[e];
        }
      }
      __syncthreads();  // barrier 5
      // Lane j of every wave holds gathered block j and learns its rank by (score desc,
      // index asc) and the mass ranked before it, so the choice reaches each thread as
      // a wave-uniform bit mask. A small bin is ranked by every wave on its own (no
      // barrier); a larger one is split over the waves, wave w comparing against
      // blocks w, w + NW, ..., and the partial counts meet in LDS (one barrier).
      const bool act = lane < C;
      const uint32_t mk = act ? sh.gk[lane] : 0u;
      const int mi = act ? sh.gi[lane] : 0x7fffffff;
      const u64 mm = act ? sh.gm[lane] : 0ull;
      int rank = 0;
      u64 cm = 0;  // mass of the blocks ranked before this one (needed for k_p only)
      if (C <= kRankRedundant && !need_kp) {
        for (int j = 0; j < C; ++j) {  // j is uniform: broadcast block j from lane j
          const uint32_t kj = __builtin_amdgcn_readlane(mk, j);
          const int ij = __builtin_amdgcn_readlane(mi, j);
          rank += (kj > mk || (kj == mk && ij < mi)) ? 1 : 0;
        }
      } else if (C <= kRankRedundant) {
        for (int j = 0; j < C; ++j) {
          const uint32_t kj = __builtin_amdgcn_readlane(mk, j);
          const int ij = __builtin_amdgcn_readlane(mi, j);
          const u64 gj = lane_value(mm, j);
          const bool before_me = kj > mk || (kj == mk && ij < mi);
          rank += before_me ? 1 : 0;
          cm += before_me ? gj : 0ull;
        }
      } else {
        for (int j = wave; j < C; j += NW) {  // uniform LDS reads are broadcasts
          const uint32_t kj = sh.gk[j];
          const int ij = sh.gi[j];
          const u64 gj = sh.gm[j];
          const bool before_me = kj > mk || (kj == mk && ij < mi);
          rank += before_me ? 1 : 0;
          cm += before_me ? gj : 0ull;
        }
        if (act) {
          atomicAdd(&sh.grank[lane], static_cast<uint32_t>(rank));
          atomicAdd(&sh.gcm[lane], cm);
        }
        __syncthreads();
        rank = static_cast<int>(sh.grank[lane]);
        cm = sh.gcm[lane];
      }
      cm += mm;  // mass of the blocks ranked at or before this one
      if (need_kp) {
        int cand = (act && PM + cm >= T) ? A + rank + 1 : 0x7fffffff;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) cand = min(cand, __shfl_xor(cand, o, 64));
        k = clampk(cand);
      }
      const bool chosen = act && rank < k - A;
      chosen_mask = __ballot(chosen);
      if (sel_mass != nullptr) {  // the chosen lanes' masses (at most C <= 64 of them)
        if (C <= kRankRedundant) {
          for (u64 bits = chosen_mask; bits != 0; bits &= bits - 1)
            inbin_mass += lane_value(mm, __builtin_ctzll(bits));
        } else {
          inbin_mass = lane_value(wave_incl_scan(chosen ? mm : 0ull), 63);
        }
      }
    } else {
      // dense boundary bin: exact radix select over the keys of that bin only
      fallback = true;
      bool act[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) act[e] = cb[e] == bk;
      u64 ca, ma, tc, tm;
      bool decided = false;
      if (need_kp) {
        const u64 tgt = T - PM;  // > 0: bin bk holds the mass crossing
        radix_select<NT, EPT, true>(key, mass, act, tgt, sh, tau, ca, ma, tc, tm);
        const u64 m_tau = tm / tc;  // every block of key tau has the same mass
        u64 c = (tgt - ma + m_tau - 1) / m_tau;
        c = c < 1 ? 1 : (c > tc ? tc : c);
        const int kp = A + static_cast<int>(ca + c);
        k = clampk(kp);
        if (k == kp) {
          take = c;
          decided = true;
        }
      }
      if (!decided) {
        radix_select<NT, EPT, false>(key, mass, act, static_cast<u64>(k - A), sh, tau, ca, ma,
                                     tc, tm);
        take = static_cast<u64>(k - A) - ca;
      }
    }
  }

  // ---- 5. membership and ascending compaction
  uint32_t tie_rank = 0;
  if (fallback) {
    uint32_t tl2 = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) tl2 += (cb[e] == bk && key[e] == tau) ? 1u : 0u;
    uint32_t tt;
    tie_rank = block_excl_scan<NT>(tl2, tt, sh.wt);
    __syncthreads();
  }
  bool sel[EPT];
  uint32_t sel_local = 0;
  u64 mass_sel = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    bool pick = false;
    if (res[e] && k > 0) {
      if (cb[e] < bk) {
        pick = true;
      } else if (cb[e] == bk) {
        if (!fallback) {
          pick = ((chosen_mask >> slot[e]) & 1ull) != 0;
        } else if (key[e] > tau) {
          pick = true;
        } else if (key[e] == tau) {
          pick = tie_rank < take;
          ++tie_rank;
        }
      }
    }
    sel[e] = (valid[e] && !res[e]) || pick;
    sel_local += sel[e] ? 1u : 0u;
    if (pick) mass_sel += mass[e];
  }
  uint32_t cnt;
  uint32_t pos = block_excl_scan<NT>(sel_local, cnt, sh.wt2);  // barrier 6
  int32_t* out = sel_idx + (size_t)b * K_max;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (sel[e]) out[pos++] = tid * EPT + e;
  }
  for (int j = static_cast<int>(cnt) + tid; j < K_max; j += NT) out[j] = -1;
  if (sel_mass != nullptr) {
    u64 ms = 0;
    if (fallback) {
      ms = block_sum<NT>(mass_sel, sh.wt);
    } else if (k > 0 && bk >= 0) {
      ms = PM + inbin_mass;
    }
    if (tid == 0)
      sel_mass[b] = Z > 0 ? static_cast<float>(static_cast<double>(ms) / static_cast<double>(Z))
                          : 0.f;
  }
  if (tid == 0) sel_cnt[b] = static_cast<int32_t>(cnt);
}

template <int NT, int EPT>
hipError_t launch_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                       float* sel_mass, int B, int nb, float p, int K_min, int K_max,
                       int n_sink, int n_rec, RowGeom geom, hipStream_t stream) {
  hipLaunchKernelGGL((select_topp_kernel<NT, EPT>), dim3(B), dim3(NT), 0, stream, scores,
                     sel_idx, sel_cnt, sel_mass, nb, p, K_min, K_max, n_sink, n_rec, geom);
  return hipGetLastError();
}

hipError_t launch_rows(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                       float* sel_mass, int B, int nb, float p, int K_min, int K_max,
                       int n_sink, int n_rec, RowGeom geom, hipStream_t stream) {
#define SPOT_TOPP(NT, EPT)                                                                  \
  return launch_topp<NT, EPT>(scores, sel_idx, sel_cnt, sel_mass, B, nb, p, K_min, K_max, \
                              n_sink, n_rec, geom, stream)
  // few blocks per thread keeps each thread's serial chain short (measured at nb 2048:
  // 512 x 4 = 6.3 us, 256 x 8 = 8.3 us, 1024 x 2 = 6.6 us)
  if (nb <= 256) SPOT_TOPP(256, 1);
  if (nb <= 512) SPOT_TOPP(512, 1);
  if (nb <= 1024) SPOT_TOPP(512, 2);
  if (nb <= 2048) SPOT_TOPP(512, 4);
  if (nb <= 4096) SPOT_TOPP(1024, 4);
  if (nb <= 8192) SPOT_TOPP(1024, 8);
  SPOT_TOPP(1024, 16);
#undef SPOT_TOPP
}

}  // namespace

hipError_t launch_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                              float* sel_mass, int B, int nb, float p, int K_min, int K_max,
                              int n_sink, int n_rec, hipStream_t stream) {
  return launch_rows(scores, sel_idx, sel_cnt, sel_mass, B, nb, p, K_min, K_max, n_sink,
                     n_rec, RowGeom{0, 0, 0, 0, 0}, stream);
}

hipError_t launch_prefill_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                                      float* sel_mass, int B, int T, int Tq, int q_pos0,
                                      int block, int nb_stride, float p, int K_min, int K_max,
                                      int n_sink, int n_rec, hipStream_t stream) {
  const int n_tiles = (T + Tq - 1) / Tq;
  return launch_rows(scores, sel_idx, sel_cnt, sel_mass, B * n_tiles, nb_stride, p, K_min,
                     K_max, n_sink, n_rec, RowGeom{n_tiles, T, Tq, q_pos0, block}, stream);
}

}  // namespace spot
