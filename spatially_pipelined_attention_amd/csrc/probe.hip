// Read-bandwidth probe: the empirical HBM bandwidth-versus-concurrency curve
// that section 4.3 of the SubGPU Pipelining paper lists among the calibration
// inputs of its search. Launched on a CU pool's stream it gives the read rate
// that pool can pull, the ceiling any stage kernel on that pool works under.
//
// Each workgroup streams its own contiguous share of the buffer once; wave w
// of a workgroup takes the 1 KB pieces w, w + 4, ... (one 16-byte load per
// lane each), with a ring of 8 pieces in flight per wave and non-temporal
// loads. The loaded values are folded into one word so the loads stay live.
#include <hip/hip_runtime.h>

#include "host.h"

namespace {

constexpr int kProbeRing = 8;

__global__ __launch_bounds__(256, 2) void k_read_probe(const char* src, long long per_wg, unsigned* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* base = src + (long long)blockIdx.x * per_wg + lane * 16;
  const int n_pieces = (int)(per_wg >> 10);
  const int nw = (n_pieces - wave + 3) / 4;   // pieces of this wave
  if (nw <= 0) return;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r[kProbeRing];
  u32x4 acc = {0u, 0u, 0u, 0u};
  auto piece = [&](int j) { return base + (long long)(wave + 4 * min(j, nw - 1)) * 1024; };
#pragma unroll
  for (int p = 0; p < kProbeRing; ++p) r[p] = __builtin_nontemporal_load((const u32x4*)piece(p));
  int i = 0;
  for (; i + kProbeRing < nw; i += kProbeRing) {
#pragma unroll
    for (int p = 0; p < kProbeRing; ++p) {
      acc ^= r[p];
      __builtin_amdgcn_sched_barrier(0);
      r[p] = __builtin_nontemporal_load((const u32x4*)piece(i + kProbeRing + p));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int p = 0; p < kProbeRing; ++p) acc ^= r[p];
  // never true for the fold of real data in practice; keeps the loads from being dropped
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9E3779B9u && lane == 0) sink[blockIdx.x & 255] = 1u;
}

}  // namespace

using namespace spa;

extern "C" spa_status spa_hbm_probe(spa_ctx* ctx, const void* src, size_t bytes, int32_t n_wgs, int32_t reps,
                                    void* stream, double* ms) {
  if (!ctx || !src || !ms || n_wgs < 1 || reps < 1 || (((uintptr_t)src) & 15))
    return fail(SPA_EINVAL, "bad argument");
  if (bytes == 0 || bytes % ((size_t)n_wgs * 1024)) return fail(SPA_EINVAL, "bytes must be a multiple of n_wgs * 1024");
  const long long per_wg = (long long)(bytes / (size_t)n_wgs);
  hipStream_t st = (hipStream_t)stream;
  unsigned* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&sink, 256 * sizeof(unsigned));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_read_probe, dim3(n_wgs), dim3(256), 0, st, (const char*)src, per_wg, sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e0, st);
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    hipLaunchKernelGGL(k_read_probe, dim3(n_wgs), dim3(256), 0, st, (const char*)src, per_wg, sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float f = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&f, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (e != hipSuccess) return hip_fail(e, "hbm probe");
  *ms = (double)f / reps;
  return SPA_OK;
}
