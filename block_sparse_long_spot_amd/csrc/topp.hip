// Dual top-p block selection (SpotAttention §2.3, Eq. 7 and Eq. 8).
//
// One work-group per query row. Every thread keeps EPT consecutive blocks in
// registers: the score, an order-preserving 32-bit key of it, and the block's
// softmax mass in 2^-38 fixed point (integer sums are exact, so nothing depends on
// the order in which threads add).
//
//   1. reserved blocks R (sink prefix, recency suffix) are set aside;
//   2. max and sum of exp(s - max) over the residual blocks (Eq. 7's softmax);
//   3. one coarse histogram of count and mass over 2048 bins of width 1/64 in
//      (max - s) (bin order = score order), turned into prefix sums. It locates the
//      bin where the cumulative mass reaches p*Z (the nucleus cut) and, because the
//      clamp k = clamp(k_p, K_min - r, K_max - r) is monotone, also decides whether
//      k is already known or falls inside that same bin;
//   4. only the bin that holds the k-th block needs an exact order: its blocks
//      (usually a handful) are gathered and one wave ranks them by (score desc,
//      index asc), accumulating mass in that order to finish k_p when needed. A bin
//      with more than 64 blocks (dense ties) falls back to an exact radix select,
//      11+11+10 bits of the key, restricted to that bin;
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

template <int NT>
struct ToppSmem {
  uint32_t hc[kCoarseBins];          // histograms (coarse pass, then the fallback passes)
  u64 hm[kCoarseBins];
  uint32_t pc[kCoarseBins + 1];      // exclusive prefix over bins: count and mass above
  u64 pm[kCoarseBins + 1];
  uint32_t gk[kRankMax];             // gathered boundary-bin blocks: key, index, mass
  int32_t gi[kRankMax];
  u64 gm[kRankMax];
  int32_t gsel[kRankMax];            // 1 if the gathered block is chosen
  int32_t ng;
  int32_t found[3];                  // bins of the mass target and two count targets
  int32_t k_final;
  u64 inbin_mass;                    // mass of the chosen blocks of the boundary bin
  u64 wa[NT / 64];
  u64 wb[NT / 64];
  float wf[NT / 64];
  uint32_t r_digit;
  u64 r_cnt_above;
  u64 r_mass_above;
};

template <int NT>
__device__ float block_max(float v, ToppSmem<NT>& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if (lane == 0) sh.wf[wave] = v;
  __syncthreads();
  float r = sh.wf[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, sh.wf[w]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ u64 block_sum(u64 v, ToppSmem<NT>& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) sh.wa[wave] = v;
  __syncthreads();
  u64 r = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) r += sh.wa[w];
  __syncthreads();
  return r;
}

// Exclusive prefix sum in thread order; also returns the total.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, ToppSmem<NT>& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wa[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = static_cast<uint32_t>(sh.wa[w]);
    if (w < wave) before += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// Radix select over the residual keys, from the largest key down.
// BY_MASS: stop where the cumulative mass reaches `target`; otherwise where the
// cumulative count does. Outputs the selected key, the count and mass strictly above
// it, and the count and mass of its tie group.
template <int NT, int EPT, bool BY_MASS>
__device__ void radix_select(const uint32_t (&key)[EPT], const u64 (&mass)[EPT],
                             const bool (&res)[EPT], u64 target, ToppSmem<NT>& sh,
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
      if (res[e] && (key[e] & pmask) == prefix) {
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
      sh.wa[wave] = sc;
      sh.wb[wave] = sm;
    }
    __syncthreads();
    u64 hc_hi = 0, hm_hi = 0;  // totals of the waves holding higher bins
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      if (w > wave) {
        hc_hi += sh.wa[w];
        hm_hi += sh.wb[w];
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

// exp(s - mx) in 2^-38 fixed point. s - mx and its split into an integer and a
// fraction are exact in fp64; only the fractional power of two is evaluated in fp32
// (about 1 ulp), so the mass carries a relative error near 1e-7.
__device__ __forceinline__ u64 fixed_mass(float s, float mx) {
  const double t = (static_cast<double>(s) - static_cast<double>(mx)) * 1.4426950408889634;
  const double n = floor(t);
  if (n < -80.0) return 0ull;
  const float f = static_cast<float>(t - n);                 // in [0, 1)
  const float v = ldexpf(exp2f(f), static_cast<int>(n) + 38);  // <= 2^38
  return static_cast<u64>(__float2ll_rn(v));
}

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void select_topp_kernel(const float* __restrict__ scores,
                                                         int32_t* __restrict__ sel_idx,
                                                         int32_t* __restrict__ sel_cnt,
                                                         float* __restrict__ sel_mass, int nb,
                                                         float p, int K_min, int K_max,
                                                         int n_sink, int n_rec) {
  constexpr int BPT = kCoarseBins / NT;
  __shared__ ToppSmem<NT> sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = scores + (size_t)b * nb;
  const int rs = min(n_sink, nb), rr = min(n_rec, nb);
  const int r = min(nb, rs + rr);
  const int n_res = nb - r;
  const int lo = max(0, K_min - r);
  const int hi_cap = min(K_max - r, n_res);  // K_max >= r is checked on the host
  // k as a function of the nucleus size: monotone in k_p
  auto clampk = [&](int x) { return min(max(x, lo), hi_cap); };

  float s[EPT];
  uint32_t key[EPT];
  bool valid[EPT], res[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid * EPT + e;
    valid[e] = i < nb;
    float v = valid[e] ? row[i] : 0.f;
    if (v == 0.f) v = 0.f;  // fold -0.0 onto +0.0
    s[e] = v;
    key[e] = float_key(v);
    res[e] = valid[e] && i >= rs && i < nb - rr;
  }
  for (int i = tid; i < kCoarseBins; i += NT) {
    sh.hc[i] = 0;
    sh.hm[i] = 0;
  }
  if (tid == 0) {
    sh.ng = 0;
    sh.found[0] = sh.found[1] = sh.found[2] = 0;
    sh.inbin_mass = 0;
  }

  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (res[e]) mx = fmaxf(mx, s[e]);
  mx = block_max<NT>(mx, sh);  // also orders the clears above

  // softmax mass in fixed point, coarse bin, histogram
  u64 mass[EPT];
  int cb[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    mass[e] = 0;
    cb[e] = -1;
    if (res[e]) {
      mass[e] = fixed_mass(s[e], mx);
      cb[e] = static_cast<int>(fminf((mx - s[e]) * kBinsPerNat, kCoarseBins - 1.f));
      atomicAdd(&sh.hc[cb[e]], 1u);
      atomicAdd(&sh.hm[cb[e]], mass[e]);
    }
  }
  __syncthreads();
  // exclusive prefix over bins in ascending bin order (= descending score)
  {
    const int b0 = tid * BPT;
    u64 lc = 0, lm = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      lc += sh.hc[b0 + i];
      lm += sh.hm[b0 + i];
    }
    u64 ic = lc, im = lm;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const u64 yc = __shfl_up(ic, o, 64);
      const u64 ym = __shfl_up(im, o, 64);
      if (lane >= o) {
        ic += yc;
        im += ym;
      }
    }
    if (lane == 63) {
      sh.wa[wave] = ic;
      sh.wb[wave] = im;
    }
    __syncthreads();
    u64 oc = 0, om = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w)
      if (w < wave) {
        oc += sh.wa[w];
        om += sh.wb[w];
      }
    u64 rc = oc + ic - lc, rm = om + im - lm;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      sh.pc[b0 + i] = static_cast<uint32_t>(rc);
      sh.pm[b0 + i] = rm;
      rc += sh.hc[b0 + i];
      rm += sh.hm[b0 + i];
    }
    if (tid == NT - 1) {
      sh.pc[kCoarseBins] = static_cast<uint32_t>(rc);
      sh.pm[kCoarseBins] = rm;
    }
    __syncthreads();
  }
  const u64 Z = sh.pm[kCoarseBins];

  // decide k, or the bin where it is decided. One pass finds the bins of the mass
  // target and of the two count targets the clamp can produce.
  int k = 0;
  int bk = -1;           // bin holding the k-th residual block in score order
  bool need_kp = false;  // k still depends on the exact nucleus size inside bin bk
  u64 T = 0;
  if (n_res > 0) {
    int tl = min(max(lo, 1), hi_cap), th = hi_cap;  // count targets (0 = none)
    if (p >= 1.f || p <= 0.f) {
      k = clampk(p >= 1.f ? n_res : 0);
      tl = k;
      th = 0;
    } else {
      T = static_cast<u64>(ceil(static_cast<double>(p) * static_cast<double>(Z)));
      if (T == 0) T = 1;
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int bb = tid * BPT + i;
      if (T > 0 && sh.pm[bb] < T && T <= sh.pm[bb + 1]) sh.found[0] = bb;
      if (sh.pc[bb] < (uint32_t)tl && (uint32_t)tl <= sh.pc[bb + 1]) sh.found[1] = bb;
      if (sh.pc[bb] < (uint32_t)th && (uint32_t)th <= sh.pc[bb + 1]) sh.found[2] = bb;
    }
    __syncthreads();
    if (T == 0) {
      if (k > 0) bk = sh.found[1];
    } else {
      const int bm = sh.found[0];
      const int A = static_cast<int>(sh.pc[bm]);
      const int C = static_cast<int>(sh.pc[bm + 1]) - A;
      const int k1 = clampk(A + 1), k2 = clampk(A + C);
      if (k1 != k2) {
        bk = bm;
        need_kp = true;
      } else {
        k = k1;
        if (k > 0) bk = k == th ? sh.found[2] : (k == tl ? sh.found[1] : bm);
      }
    }
  }

  // exact order inside the boundary bin
  uint32_t tau = 0;
  u64 take = 0;  // fallback: blocks of key tau to take, lowest index first
  int slot[EPT];
  bool fallback = false;
  if (bk >= 0) {
    const int A = static_cast<int>(sh.pc[bk]);
    const int C = static_cast<int>(sh.pc[bk + 1]) - A;
    if (C <= kRankMax) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        slot[e] = -1;
        if (cb[e] == bk) {
          const int sl = atomicAdd(&sh.ng, 1);
          slot[e] = sl;
          sh.gk[sl] = key[e];
          sh.gi[sl] = tid * EPT + e;
          sh.gm[sl] = mass[e];
        }
      }
      __syncthreads();
      if (wave == 0) {
        const bool act = lane < C;
        const uint32_t mk = act ? sh.gk[lane] : 0u;
        const int mi = act ? sh.gi[lane] : 0x7fffffff;
        const u64 mm = act ? sh.gm[lane] : 0ull;
        const uint32_t mlo = static_cast<uint32_t>(mm), mhi = static_cast<uint32_t>(mm >> 32);
        int rank = 0;
        u64 cm = mm;  // mass of the blocks ranked at or before this one
        for (int j = 0; j < C; ++j) {  // j is uniform: broadcast block j from lane j
          const uint32_t kj = __builtin_amdgcn_readlane(mk, j);
          const int ij = __builtin_amdgcn_readlane(mi, j);
          const u64 gj = (static_cast<u64>(__builtin_amdgcn_readlane(mhi, j)) << 32) |
                         __builtin_amdgcn_readlane(mlo, j);
          const bool before = kj > mk || (kj == mk && ij < mi);
          rank += before ? 1 : 0;
          cm += before ? gj : 0ull;
        }
        int kk = k;
        if (need_kp) {
          int cand = (act && sh.pm[bk] + cm >= T) ? A + rank + 1 : 0x7fffffff;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) cand = min(cand, __shfl_xor(cand, o, 64));
          kk = clampk(cand);
        }
        const bool chosen = act && rank < kk - A;
        if (act) sh.gsel[lane] = chosen ? 1 : 0;
        u64 im = chosen ? mm : 0ull;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) im += __shfl_xor(im, o, 64);
        if (lane == 0) {
          sh.k_final = kk;
          sh.inbin_mass = im;
        }
      }
      __syncthreads();
      k = sh.k_final;
    } else {
      // dense boundary bin: exact radix select over the keys of that bin only
      fallback = true;
      bool act[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) act[e] = cb[e] == bk;
      u64 ca, ma, tc, tm;
      bool decided = false;
      if (need_kp) {
        const u64 tgt = T - sh.pm[bk];  // > 0: bin bk holds the mass crossing
        radix_select<NT, EPT, true>(key, mass, act, tgt, sh, tau, ca, ma, tc, tm);
        const u64 m_tau = tm / tc;      // every block of key tau has the same mass
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

  // membership: earlier bins, the chosen blocks of bin bk, and the reserved set
  uint32_t tie_rank = 0;
  if (fallback) {
    uint32_t tl = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) tl += (cb[e] == bk && key[e] == tau) ? 1u : 0u;
    uint32_t tt;
    tie_rank = block_excl_scan<NT>(tl, tt, sh);
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
          pick = sh.gsel[slot[e]] != 0;
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
  uint32_t pos = block_excl_scan<NT>(sel_local, cnt, sh);
  int32_t* out = sel_idx + (size_t)b * K_max;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (sel[e]) out[pos++] = tid * EPT + e;
  }
  for (int j = static_cast<int>(cnt) + tid; j < K_max; j += NT) out[j] = -1;
  if (sel_mass != nullptr) {
    u64 ms = 0;
    if (k > 0 && bk >= 0) ms = fallback ? block_sum<NT>(mass_sel, sh) : sh.pm[bk] + sh.inbin_mass;
    if (tid == 0)
      sel_mass[b] = Z > 0 ? static_cast<float>(static_cast<double>(ms) / static_cast<double>(Z))
                          : 0.f;
  }
  if (tid == 0) sel_cnt[b] = static_cast<int32_t>(cnt);
}

template <int NT, int EPT>
hipError_t launch_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                       float* sel_mass, int B, int nb, float p, int K_min, int K_max,
                       int n_sink, int n_rec, hipStream_t stream) {
  hipLaunchKernelGGL((select_topp_kernel<NT, EPT>), dim3(B), dim3(NT), 0, stream, scores,
                     sel_idx, sel_cnt, sel_mass, nb, p, K_min, K_max, n_sink, n_rec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_topp(const float* scores, int32_t* sel_idx, int32_t* sel_cnt,
                              float* sel_mass, int B, int nb, float p, int K_min, int K_max,
                              int n_sink, int n_rec, hipStream_t stream) {
#define SPOT_TOPP(NT, EPT)                                                                  \
  return launch_topp<NT, EPT>(scores, sel_idx, sel_cnt, sel_mass, B, nb, p, K_min, K_max, \
                              n_sink, n_rec, stream)
  if (nb <= 256) SPOT_TOPP(256, 1);
  if (nb <= 512) SPOT_TOPP(256, 2);
  if (nb <= 1024) SPOT_TOPP(256, 4);
  if (nb <= 2048) SPOT_TOPP(256, 8);
  if (nb <= 4096) SPOT_TOPP(256, 16);
  if (nb <= 8192) SPOT_TOPP(1024, 8);
  SPOT_TOPP(1024, 16);
#undef SPOT_TOPP
}

}  // namespace spot
