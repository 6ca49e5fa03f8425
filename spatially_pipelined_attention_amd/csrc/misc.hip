// Small kernels of the decode layer on gfx950: the MoE combine + residual
// (Figure 3 "Combine" of the SubGPU Pipelining paper) with the row
// sum-of-squares the next RMSNorm needs, per-row fp8 activation quantisation,
// KV cache row I/O, counter clears and a CU placement probe.
#include "common.h"
#include "kernels.h"

namespace spa {

// x_out[t] = h[t] + sum_{s < k} w[t][s] * y[inv[t][s]] (pick order, fp32);
// ss_out[tile][t] = sum over the tile's 64 columns of x_out^2.
// One wave per (token, 64-column tile); lane = column.
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_tiles = a.H >> 6;
  const int tile = blockIdx.x * 4 + wave;
  const int t = blockIdx.y;
  if (tile >= n_tiles) return;
  const int col = tile * 64 + lane;
  float v = a.h[(long long)t * a.H + col];
  for (int s = 0; s < a.k; ++s) {
    const float w = a.w[t * a.k + s];
    const int row = a.inv[t * a.k + s];
    v += w * a.y[(long long)row * a.H + col];
  }
  a.x_out[(long long)t * a.H + col] = v;
  const float ss = wave_sum(v * v);
  if (lane == 0) a.ss_out[(long long)tile * a.ss_ld + t] = ss;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const int n_tiles = a.H / 64;
  dim3 grid((n_tiles + 3) / 4, a.n_tok);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// One workgroup per row: v = x * rstd * gamma (or x), s = smallest power of
// two with max|v| <= 448 s, codes = E4M3(v / s).
__global__ __launch_bounds__(256) void k_quant_e4m3(QuantArgs a) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  if (a.n_rows_dev && r >= *a.n_rows_dev) return;
  const int src = a.row_src ? a.row_src[r] : r;
  const float* x = a.x + (long long)src * a.x_ld;
  float rstd = 1.f;
  if (a.ss) {
    float ssum = 0.f;
    for (int t = 0; t < a.ss_tiles; ++t) ssum += a.ss[(long long)t * a.ss_ld + src];
    rstd = 1.0f / sqrtf(ssum * a.inv_h + a.eps);
  }
  float amax = 0.f;
  for (int c = threadIdx.x; c < a.n_cols; c += 256) {
    float v = x[c] * rstd;
    if (a.gamma) v *= a.gamma[c];
    amax = fmaxf(amax, fabsf(v));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // smallest power of two s with amax <= 448 * s
  float s = 1.f;
  if (amax > 0.f) {
    int e;
    frexpf(amax / 448.0f, &e);            // amax/448 in [2^(e-1), 2^e)
    s = ldexpf(1.f, e);
    if (amax <= 448.0f * ldexpf(1.f, e - 1)) s = ldexpf(1.f, e - 1);
  }
  if (threadIdx.x == 0) a.scales[r] = s;
  const float inv_s = 1.0f / s;           // exact: power of two
  uint8_t* o = a.codes + (long long)r * a.n_cols;
  for (int c = threadIdx.x; c < a.n_cols; c += 256) {
    float v = x[c] * rstd;
    if (a.gamma) v *= a.gamma[c];
    o[c] = f32_to_e4m3(v * inv_s);
  }
}

hipError_t launch_quant_e4m3(const QuantArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_e4m3, dim3(a.n_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

__global__ void k_fill_i32(int* p, long long n, int v) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int* p, long long n, int v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(k_fill_i32, dim3((int)g), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// KV cache rows <-> [n][Hkv][D] (one (sequence, position) per row, all KV heads).
// Thread -> (row, head, d).
__global__ void k_kv_io(KvIoArgs a) {
  const long long total = (long long)a.n * a.n_kv_heads * a.head_dim;
  const int D = a.head_dim;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int d = (int)(i % D);
    const long long rh = i / D;
    const int g = (int)(rh % a.n_kv_heads);
    const int r = (int)(rh / a.n_kv_heads);
    const int seq = a.seq[r], pos = a.pos[r];
    if (seq < 0 || seq >= a.n_seq || pos < 0) continue;
    long long base;
    int slot;
    if (a.kv_kind == KV_RING) {
      base = ((long long)seq * a.n_kv_heads + g) * a.window * D;
      slot = pos % a.window;
    } else {
      if (pos < 0 || pos >= a.kv_cap[seq]) continue;
      base = (a.kv_off[seq] * a.n_kv_heads + (long long)g * a.kv_cap[seq]) * D;
      slot = pos;
    }
    const long long ko = base + (long long)slot * D + d;
    const long long vo = base + (long long)(slot >> 5) * 32 * D + (long long)d * 32 + v_slot(slot & 31);
    if (a.kv_dtype == DT_BF16) {
      uint16_t* kc = (uint16_t*)a.k_cache;
      uint16_t* vc = (uint16_t*)a.v_cache;
      uint16_t* kr = (uint16_t*)a.k_rows;
      uint16_t* vr = (uint16_t*)a.v_rows;
      if (a.write) { kc[ko] = kr[i]; vc[vo] = vr[i]; }
      else { kr[i] = kc[ko]; vr[i] = vc[vo]; }
    } else {
      float* kc = (float*)a.k_cache;
      float* vc = (float*)a.v_cache;
      float* kr = (float*)a.k_rows;
      float* vr = (float*)a.v_rows;
      if (a.write) { kc[ko] = kr[i]; vc[vo] = vr[i]; }
      else { kr[i] = kc[ko]; vr[i] = vc[vo]; }
    }
  }
}

hipError_t launch_kv_io(const KvIoArgs& a, hipStream_t st) {
  const long long total = (long long)a.n * a.n_kv_heads * a.head_dim;
  if (total <= 0) return hipSuccess;
  long long g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_kv_io, dim3((int)g), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Each workgroup spins briefly (so that many are resident at once) and then
// records the hardware ids of the CU it ran on: XCC_ID and HW_ID (SE/SH/CU).
__global__ void k_probe(unsigned* out, int spin) {
  if (threadIdx.x != 0) return;
  unsigned xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11));   // HW_REG_XCC_ID bits [3:0]
  unsigned hw = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));     // HW_REG_HW_ID
  long long t0 = clock64();
  while (clock64() - t0 < spin) {
  }
  out[2 * blockIdx.x + 0] = xcc;
  out[2 * blockIdx.x + 1] = hw;
}

hipError_t launch_probe(unsigned* out, int n_blocks, int spin, hipStream_t st) {
  hipLaunchKernelGGL(k_probe, dim3(n_blocks), dim3(64), 0, st, out, spin);
  return hipGetLastError();
}

}  // namespace spa
