// Dual top-p block selection (SpotAttention §2.3, Eq. 7 and Eq. 8).
//
// One work-group per query row. Every thread keeps EPT consecutive blocks in
// registers, as an order-preserving 32-bit key of the score and the block's softmax
// mass in 2^-38 fixed point (integer sums are exact, so the selection never depends
// on the order in which threads add).
//
//   1. reserved blocks R (sink prefix, recency suffix) are set aside;
//   2. max and sum of exp(s - max) over the residual blocks (Eq. 7's softmax);
//   3. k_p: a radix select over the keys, 11+11+10 bits from the top, with a count and
//      a mass histogram per pass, finds the key tau at which the cumulative mass in
//      (score desc) order first reaches p*Z; inside tau's tie group the mass is equal
//      per block, so the number of tied blocks needed is a division;
//   4. k = clamp(k_p, K_min - r, K_max - r); if the clamp moved k, a count-only
//      radix select finds the k-th key instead;
//   5. blocks above tau, and the lowest-index tied blocks, join R; a block-wide scan
//      writes them in ascending order.
#include "device_common.h"
#include "spot_internal.h"

namespace spot {
namespace {

typedef unsigned long long u64;
constexpr double kMassOne = 274877906944.0;  // 2^38: fixed-point unit of softmax mass

template <int NT>
struct ToppSmem {
  uint32_t hc[2048];
  u64 hm[2048];
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

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void select_topp_kernel(const float* __restrict__ scores,
                                                         int32_t* __restrict__ sel_idx,
                                                         int32_t* __restrict__ sel_cnt,
                                                         float* __restrict__ sel_mass, int nb,
                                                         float p, int K_min, int K_max,
                                                         int n_sink, int n_rec) {
  __shared__ ToppSmem<NT> sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = scores + (size_t)b * nb;
  const int rs = min(n_sink, nb), rr = min(n_rec, nb);
  const int r = min(nb, rs + rr);
  const int n_res = nb - r;

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

  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (res[e]) mx = fmaxf(mx, s[e]);
  mx = block_max<NT>(mx, sh);

  u64 mass[EPT];
  u64 zl = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    mass[e] = res[e] ? static_cast<u64>(__double2ll_rn(
                           exp(static_cast<double>(s[e]) - static_cast<double>(mx)) * kMassOne))
                     : 0ull;
    zl += mass[e];
  }
  const u64 Z = block_sum<NT>(zl, sh);

  // nucleus size k_p
  int k_p = 0;
  bool have_mass_cut = false;
  uint32_t tau = 0;
  u64 take = 0;
  if (n_res > 0) {
    if (p >= 1.f) {
      k_p = n_res;
    } else if (p > 0.f) {
      const double T = static_cast<double>(p) * static_cast<double>(Z);
      u64 target = static_cast<u64>(ceil(T));
      if (target == 0) target = 1;
      u64 ca, ma, tc, tm;
      radix_select<NT, EPT, true>(key, mass, res, target, sh, tau, ca, ma, tc, tm);
      const u64 m_tau = tm / tc;  // every tied block has the same mass
      u64 c = (target - ma + m_tau - 1) / m_tau;
      if (c < 1) c = 1;
      if (c > tc) c = tc;
      k_p = static_cast<int>(ca + c);
      take = c;
      have_mass_cut = true;
    }
  }
  const int lo = max(0, K_min - r);
  const int hi = K_max - r;
  const int k = min(min(max(k_p, lo), hi), n_res);
  if (k > 0 && !(have_mass_cut && k == k_p)) {
    u64 ca, ma, tc, tm;
    radix_select<NT, EPT, false>(key, mass, res, static_cast<u64>(k), sh, tau, ca, ma, tc, tm);
    take = static_cast<u64>(k) - ca;
  }

  // rank of each tied block among the tie group, in index order
  uint32_t tie_local = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) tie_local += (k > 0 && res[e] && key[e] == tau) ? 1u : 0u;
  uint32_t tie_total;
  uint32_t tie_rank = block_excl_scan<NT>(tie_local, tie_total, sh);

  bool sel[EPT];
  uint32_t sel_local = 0;
  u64 mass_sel = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const bool reserved = valid[e] && !res[e];
    bool pick = false;
    if (k > 0 && res[e]) {
      if (key[e] > tau) {
        pick = true;
      } else if (key[e] == tau) {
        pick = tie_rank < take;
        ++tie_rank;
      }
    }
    sel[e] = reserved || pick;
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
    const u64 ms = block_sum<NT>(mass_sel, sh);
    if (tid == 0) sel_mass[b] = Z > 0 ? static_cast<float>(static_cast<double>(ms) /
                                                          static_cast<double>(Z))
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
