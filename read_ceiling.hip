// Read-bandwidth and launch-floor references for the benchmark (not part of the decode
// path).
//
// A kernel that does nothing but read: n_blocks 16 KiB blocks of a device buffer, in the
// order a block list gives, 16-byte non-temporal loads, each work-group taking an equal
// share of the list. Timed over the same byte count and block granularity as a decode
// step's K/V gather (a 64-token block of one KV head at d = 128 in bf16 is 16 KiB), it
// measures the rate this part sustains for that access pattern with no compute at all,
// which bounds what the attention kernel can reach.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kBlockVec = 16384 / 16;  // 16-byte vectors per block

__global__ __launch_bounds__(kThreads) void read_blocks(const u32x4* __restrict__ base,
                                                        const int32_t* __restrict__ list,
                                                        int per_wg, unsigned* __restrict__ sink) {
  unsigned acc = 0;
  // two blocks (8 loads per thread) in flight per step
  for (int i = 0; i < per_wg; i += 2) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4* b = base + (size_t)list[(size_t)blockIdx.x * per_wg + i + u] * kBlockVec +
                       threadIdx.x;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[u * 4 + k] = __builtin_nontemporal_load(b + k * kThreads);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  // a data-dependent store the compiler cannot drop (the value is essentially never hit)
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// Launch-floor probes: an empty kernel, and one that reads and writes one float per
// thread (a kernel with one memory round trip and nothing else).
__global__ void empty_kernel() {}

__global__ __launch_bounds__(kThreads) void touch_kernel(const float* __restrict__ a,
                                                         float* __restrict__ b, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) b[i] = a[i] * 2.f;
}

}  // namespace

extern "C" {

// Reads blocks list[0 .. n_blocks) (each an index of a 16 KiB block of `base`) with
// `wgs` work-groups of 256 threads on `stream`. n_blocks must be a positive multiple of
// 2 * wgs; `sink` must hold wgs words. Returns 0, or -1 on a bad argument (nothing
// launched). The caller keeps every index below the buffer's block count.
__attribute__((visibility("default"))) int spot_probe_read_blocks(const void* base,
                                                                  const int32_t* list,
                                                                  int n_blocks, int wgs,
                                                                  unsigned* sink,
                                                                  hipStream_t stream) {
  if (!base || !list || !sink || wgs <= 0 || n_blocks <= 0 || n_blocks % (2 * wgs) != 0)
    return -1;
  hipLaunchKernelGGL(read_blocks, dim3(wgs), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(base), list, n_blocks / wgs, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Launches `reps` empty kernels of `wgs` work-groups of 256 threads back to back on
// `stream`. Returns 0, or -1 on a bad argument (nothing launched).
__attribute__((visibility("default"))) int spot_probe_empty(int wgs, int reps,
                                                            hipStream_t stream) {
  if (wgs <= 0 || reps <= 0) return -1;
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(empty_kernel, dim3(wgs), dim3(kThreads), 0, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Launches `reps` kernels back to back on `stream`, each setting b[i] = 2 a[i] for
// i < n (one thread per element). a and b hold at least n floats.
__attribute__((visibility("default"))) int spot_probe_touch(const float* a, float* b, int n,
                                                            int reps, hipStream_t stream) {
  if (!a || !b || n <= 0 || reps <= 0) return -1;
  const int wgs = (n + kThreads - 1) / kThreads;
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(touch_kernel, dim3(wgs), dim3(kThreads), 0, stream, a, b, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
