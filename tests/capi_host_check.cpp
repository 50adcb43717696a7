// Host-only check of libspot's C ABI argument validation, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_capi_sanitized.py (g++, no GPU).
//
// The real capi.cpp and the real split plan (attn_plan.cpp) are linked against the stub
// launchers below, which only record that they were called and with which sizes. Every
// entry point is called with a valid argument set (it must return SPOT_OK and launch
// once) and with one bad argument at a time (it must return the documented error and
// launch nothing), including sizes near the int limits the checks guard against.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "spot.h"
#include "spot_internal.h"

namespace {
int g_launches = 0;
long g_last_B = 0;
}  // namespace

namespace spot {
hipError_t launch_select_score(const void*, int, const void*, const float*, const void*,
                               const void*, int, float*, int B, int, int, int, int,
                               hipStream_t) {
  ++g_launches;
  g_last_B = B;
  return hipSuccess;
}
hipError_t launch_quantize_selector(const void*, bool, int, void*, void*, const float*,
                                    long n_groups, hipStream_t) {
  ++g_launches;
  g_last_B = n_groups;
  return hipSuccess;
}
hipError_t launch_prefill_select_topp(const float*, int32_t*, int32_t*, float*, int B, int,
                                      int, int, int, int, float, int, int, int, int,
                                      hipStream_t) {
  ++g_launches;
  g_last_B = B;
  return hipSuccess;
}
hipError_t launch_select_topp(const float*, int32_t*, int32_t*, float*, int B, int, float,
                              int, int, int, int, hipStream_t) {
  ++g_launches;
  g_last_B = B;
  return hipSuccess;
}
hipError_t noalloc_scratch(hipStream_t, void** ptr) {
  *ptr = reinterpret_cast<void*>(0x40000);
  return hipSuccess;
}
hipError_t launch_sparse_attn(const void*, const void*, const void*, bool, const int32_t*,
                              const int32_t*, int, void*, void*, int B, int, int, int, int, int,
                              float, hipStream_t) {
  ++g_launches;
  g_last_B = B;
  return hipSuccess;
}
hipError_t launch_prefill_select_score(const void*, const float*, const void*, const void*,
                                       int, float*, int B, int, int, int, int, int, int, int,
                                       int, int, hipStream_t) {
  ++g_launches;
  g_last_B = B;
  return hipSuccess;
}
hipError_t launch_prefill_attn(const void*, const void*, const void*, const int32_t*,
                               const int32_t*, int, void*, int B, int, int, int, int, int, int,
                               int, float, hipStream_t) {
  ++g_launches;
  g_last_B = B;
  return hipSuccess;
}
}  // namespace spot

namespace {

int failures = 0;

// Runs `call`, expects status `want` and `launches` new launches.
template <typename F>
void expect(const char* what, int want, int launches, F call) {
  const int before = g_launches;
  const int got = call();
  const int n = g_launches - before;
  if (got != want || n != launches) {
    printf("FAIL %s: status %d (want %d), launches %d (want %d)\n", what, got, want, n,
           launches);
    ++failures;
  }
}

void* P(uintptr_t a = 0x10000) { return reinterpret_cast<void*>(a); }
float* F(uintptr_t a = 0x10000) { return reinterpret_cast<float*>(a); }
int32_t* I(uintptr_t a = 0x10000) { return reinterpret_cast<int32_t*>(a); }

struct Score {
  const void* q = P();
  int qd = SPOT_BF16;
  const void* qs = nullptr;
  const float* w = F();
  const void* k = P();
  const void* ks = nullptr;
  int kd = SPOT_BF16;
  float* s = F();
  int B = 8, nb = 2048, kpb = 1, H = 4, di = 64;
  int operator()() const {
    return spot_select_score(q, qd, qs, w, k, ks, kd, s, B, nb, kpb, H, di, nullptr);
  }
};

struct Topp {
  const float* s = F();
  int32_t* idx = I();
  int32_t* cnt = I();
  float* mass = nullptr;
  int B = 8, nb = 2048;
  float p = 0.95f;
  int K_min = 16, K_max = 256, n_sink = 1, n_rec = 4;
  int operator()() const {
    return spot_select_topp(s, idx, cnt, mass, B, nb, p, K_min, K_max, n_sink, n_rec, nullptr);
  }
};

struct Attn {
  const void* q = P();
  const void* k = P();
  const void* v = P();
  int dt = SPOT_BF16;
  const int32_t* idx = I();
  const int32_t* cnt = I();
  int K_max = 256;
  void* out = P();
  void* ws = P();
  size_t ws_bytes = (size_t)1 << 40;
  int B = 8, Hq = 32, Hkv = 8, d = 128, L = 131072, block = 64;
  float scale = 0.088f;
  int operator()() const {
    return spot_sparse_attn(q, k, v, dt, idx, cnt, K_max, out, ws, ws_bytes, B, Hq, Hkv, d, L,
                            block, scale, nullptr);
  }
  int noalloc() const {
    return spot_sparse_attn_noalloc(q, k, v, dt, idx, cnt, K_max, out, B, Hq, Hkv, d, L, block,
                                    scale, nullptr);
  }
};

struct Quant {
  const void* src = P();
  int sd = SPOT_BF16, rows = 131072, len = 512, fmt = SPOT_INT4_G32;
  void* codes = P();
  void* scales = P();
  const float* ts = nullptr;
  int operator()() const {
    return spot_quantize_selector(src, sd, rows, len, fmt, codes, scales, ts, nullptr);
  }
};

struct PScore {
  const void* q = P();
  int qd = SPOT_BF16;
  const float* w = F();
  const void* k = P();
  const void* ks = nullptr;
  int kd = SPOT_BF16;
  float* s = F();
  int B = 1, T = 32768, Tq = 128, pos0 = 0, nb_cache = 512, kpb = 1, H = 4, di = 64,
      block = 64;
  int operator()() const {
    return spot_prefill_select_score(q, qd, w, k, ks, kd, s, B, T, Tq, pos0, nb_cache, kpb, H,
                                     di, block, nullptr);
  }
};

struct PTopp {
  const float* s = F();
  int32_t* idx = I();
  int32_t* cnt = I();
  float* mass = nullptr;
  int B = 1, T = 32768, Tq = 128, pos0 = 0, block = 64;
  float p = 0.95f;
  int K_min = 0, K_max = 512, n_sink = 1, n_rec = 4;
  int operator()() const {
    return spot_prefill_select_topp(s, idx, cnt, mass, B, T, Tq, pos0, block, p, K_min, K_max,
                                    n_sink, n_rec, nullptr);
  }
};

struct PAttn {
  const void* q = P();
  const void* k = P();
  const void* v = P();
  int dt = SPOT_BF16;
  const int32_t* idx = I();
  const int32_t* cnt = I();
  int K_max = 512;
  void* out = P();
  int B = 1, Hq = 32, Hkv = 8, T = 32768, Tq = 128, pos0 = 0, d = 128, L = 32768, block = 64;
  float scale = 0.088f;
  int operator()() const {
    return spot_prefill_attn(q, k, v, dt, idx, cnt, K_max, out, B, Hq, Hkv, T, Tq, pos0, d, L,
                             block, scale, nullptr);
  }
};

}  // namespace

int main() {
  const int OK = SPOT_OK, INV = SPOT_ERR_INVALID, UNS = SPOT_ERR_UNSUPPORTED;
  const int big = 2147483647;

  // ---- spot_select_score
  expect("score ok", OK, 1, Score{});
  expect("score null q", INV, 0, [] { Score a; a.q = nullptr; return a(); });
  expect("score misaligned k", INV, 0, [] { Score a; a.k = P(0x10008); return a(); });
  expect("score B 0", INV, 0, [] { Score a; a.B = 0; return a(); });
  expect("score kpb -1", INV, 0, [] { Score a; a.kpb = -1; return a(); });
  expect("score unknown format", INV, 0, [] { Score a; a.kd = 9; return a(); });
  expect("score int4 no scale", INV, 0, [] { Score a; a.kd = SPOT_INT4_G32; return a(); });
  expect("score d_idx 96", UNS, 0, [] { Score a; a.di = 96; return a(); });
  expect("score B 65536", UNS, 0, [] { Score a; a.B = 65536; return a(); });
  expect("score nb max", OK, 1, [] { Score a; a.B = 1; a.nb = big; a.kpb = big; return a(); });

  // ---- spot_select_topp
  expect("topp ok", OK, 1, Topp{});
  expect("topp nan p", INV, 0, [] { Topp a; a.p = NAN; return a(); });
  expect("topp K_max < r", INV, 0, [] { Topp a; a.K_max = 4; return a(); });
  expect("topp sink > nb, K_max < nb", INV, 0, [] {
    Topp a; a.n_sink = big; a.n_rec = big; a.K_max = 2047; return a(); });
  expect("topp sink and rec near int max", OK, 1, [] {
    Topp a; a.n_sink = big; a.n_rec = big; a.K_max = 2048; return a(); });
  expect("topp nb 16385", UNS, 0, [] { Topp a; a.nb = 16385; a.K_max = 20000; return a(); });
  expect("topp B max", UNS, 0, [] { Topp a; a.B = big; return a(); });
  expect("topp misaligned mass", INV, 0, [] { Topp a; a.mass = F(0x10002); return a(); });

  // ---- spot_sparse_attn and the allocation-free form
  {
    Attn a;
    a.ws_bytes = spot_sparse_attn_workspace_bytes(a.B, a.Hq, a.Hkv, a.d, a.K_max, a.block, a.dt);
    expect("attn exact workspace", OK, 1, a);
    Attn s = a;
    s.ws_bytes -= 1;
    expect("attn workspace one short", INV, 0, s);
  }
  expect("attn null ws", INV, 0, [] { Attn a; a.ws = nullptr; return a(); });
  expect("attn misaligned ws", INV, 0, [] { Attn a; a.ws = P(0x10080); return a(); });
  expect("attn Hq % Hkv", INV, 0, [] { Attn a; a.Hq = 30; return a(); });
  expect("attn inf scale", INV, 0, [] { Attn a; a.scale = INFINITY; return a(); });
  expect("attn block 256", UNS, 0, [] { Attn a; a.block = 256; return a(); });
  expect("attn G 16", UNS, 0, [] { Attn a; a.Hq = 128; return a(); });
  expect("attn B 65536", UNS, 0, [] { Attn a; a.B = 65536; return a(); });
  expect("attn B*Hq overflow", UNS, 0, [] { Attn a; a.B = 65535; a.Hq = 65536; a.Hkv = 8192;
                                            return a(); });
  expect("attn K_max max", OK, 1, [] { Attn a; a.K_max = big; a.ws_bytes = SIZE_MAX;
                                        return a(); });
  expect("attn K_max max, 1 TiB workspace", INV, 0, [] { Attn a; a.K_max = big; return a(); });
  expect("attn L max", OK, 1, [] { Attn a; a.L = big; return a(); });
  expect("noalloc ok", OK, 1, [] { Attn a; return a.noalloc(); });
  expect("noalloc too big", UNS, 0, [] { Attn a; a.B = 64; return a.noalloc(); });
  expect("noalloc null q", INV, 0, [] { Attn a; a.q = nullptr; return a.noalloc(); });
  if (spot_sparse_attn_workspace_bytes(8, 32, 8, 128, 256, 48, SPOT_BF16) != 0 ||
      spot_sparse_attn_workspace_bytes(8, 32, 8, 128, 256, 64, 7) != 0 ||
      spot_sparse_attn_workspace_bytes(-1, 32, 8, 128, 256, 64, SPOT_BF16) != 0) {
    printf("FAIL workspace size of invalid arguments\n");
    ++failures;
  }
  // every supported block and batch: the plan keeps the workspace finite and positive
  for (int block : {16, 32, 64, 128})
    for (int B : {1, 2, 7, 64, 65, 4096})
      for (int K : {1, 256, 8192, 65536}) {
        const size_t w = spot_sparse_attn_workspace_bytes(B, 32, 8, 128, K, block, SPOT_BF16);
        const size_t f = spot_sparse_attn_workspace_bytes(B, 32, 8, 128, K, block, SPOT_F32);
        if (w == 0 || f == 0) {
          printf("FAIL workspace 0 at block %d B %d K %d\n", block, B, K);
          ++failures;
        }
      }

  // ---- spot_quantize_selector
  expect("quant ok", OK, 1, Quant{});
  expect("quant row_len 48", INV, 0, [] { Quant a; a.len = 48; return a(); });
  expect("quant int8 with group scales", INV, 0, [] {
    Quant a; a.fmt = SPOT_INT8; a.ts = F(); return a(); });
  expect("quant many groups", UNS, 0, [] { Quant a; a.rows = big; a.len = big - 31; return a(); });

  // ---- prefill
  expect("prefill score ok", OK, 1, PScore{});
  expect("prefill score nb_cache short", INV, 0, [] { PScore a; a.nb_cache = 511; return a(); });
  expect("prefill score pos0 + T overflow", INV, 0, [] {
    PScore a; a.pos0 = big; a.nb_cache = big; return a(); });
  expect("prefill score fp32", UNS, 0, [] { PScore a; a.qd = SPOT_F32; return a(); });
  expect("prefill score fp32 keys", UNS, 0, [] { PScore a; a.kd = SPOT_F32; return a(); });
  expect("prefill score int4 keys", OK, 1, [] { PScore a; a.kd = SPOT_INT4_G32; a.ks = P();
                                                return a(); });
  expect("prefill score int4 keys without scales", INV, 0, [] { PScore a; a.kd = SPOT_INT4_G32;
                                                                return a(); });
  expect("prefill topp ok", OK, 1, PTopp{});
  expect("prefill topp K_max < r", INV, 0, [] { PTopp a; a.K_max = 4; return a(); });
  expect("prefill topp long", UNS, 0, [] { PTopp a; a.T = big - 64; return a(); });
  expect("prefill topp pos0 + T overflow", INV, 0, [] { PTopp a; a.pos0 = big; return a(); });
  expect("prefill attn ok", OK, 1, PAttn{});
  expect("prefill attn past L", INV, 0, [] { PAttn a; a.pos0 = 1; return a(); });
  expect("prefill attn pos0 + T overflow", INV, 0, [] { PAttn a; a.pos0 = big; return a(); });
  expect("prefill attn d 64", UNS, 0, [] { PAttn a; a.d = 64; return a(); });
  expect("prefill attn K_max 8193", UNS, 0, [] { PAttn a; a.K_max = 8193; return a(); });

  if (spot_abi_version() != 3) {
    printf("FAIL abi version %d\n", spot_abi_version());
    ++failures;
  }
  for (int st : {0, -1, -2, -3, 5})
    if (!spot_status_string(st) || !spot_status_string(st)[0]) ++failures;

  printf("%s: %d failure(s)\n", failures ? "FAILED" : "passed", failures);
  return failures ? 1 : 0;
}
