// Row-wise kernels of the decode layer on gfx950 (Figure 3 of the SubGPU
// Pipelining paper): they finish the split products, one workgroup per token
// row, and fuse the light operators that need whole rows:
//   k_qkv_finish   - sum of the QKV splits -> q, and the new K/V written into
//                    the cache slot of position L-1 ("KV proj" + append),
//                    with the rotary embedding of q and k ("RoPE") when set;
//   k_oproj_finish - residual add of the output projection ("Add+Norm"), the
//                    RMSNorm statistic, and the normalised row in fp32 (router
//                    input), bf16 and power-of-two-scaled E4M3 (expert input);
//   k_route_topk   - router logits, top-k in logit order (ties to the lower
//                    index) and softmax over the picks, one wave per token;
//   k_route_permute- the dispatch permutation (counts, offsets, rows grouped
//                    by expert with (token, pick) ascending inside, inverse),
//                    run by the last k_route_topk_perm workgroup to finish,
//                    or as its own launch where it also gathers the rows;
//   k_combine      - "Combine": weighted sum of the expert outputs in pick
//                    order plus residual, and the next layer's RMSNorm;
// plus row conversion, KV row I/O, counter fill and a CU placement probe.
// Every reduction runs in a fixed order, so results never depend on timing.
#include <algorithm>

#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace spa {

constexpr int kRowThreads = 1024;   // row kernels: one workgroup per token row
constexpr int kRowCols = 4;         // columns per thread: rows up to 4096 wide

// Deterministic sum / max over a kRowThreads workgroup (fixed tree order).
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kRowThreads / 64; ++w) t += red[w];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) t = fmaxf(t, red[w]);
  return t;
}

constexpr int kMaxSplits = 16;   // plan_gemm never splits k more than this

// Kernels that sum split partials (part_sum) take SM, a compile-time bound on
// the split count, so that all SM loads are issued before the first add; they
// are instantiated for SM = 1, 2, 4, 8, 16 and launched with the smallest
// bound that holds: KERNEL<SM> with the smallest SM >= S.
#define SPA_LAUNCH_SPLITS(S, KERNEL, GRID, BLOCK, LDS, ST, ...)                      \
  do {                                                                               \
    if ((S) <= 1) hipLaunchKernelGGL((KERNEL<1>), GRID, BLOCK, LDS, ST, __VA_ARGS__);      \
    else if ((S) <= 2) hipLaunchKernelGGL((KERNEL<2>), GRID, BLOCK, LDS, ST, __VA_ARGS__); \
    else if ((S) <= 4) hipLaunchKernelGGL((KERNEL<4>), GRID, BLOCK, LDS, ST, __VA_ARGS__); \
    else if ((S) <= 8) hipLaunchKernelGGL((KERNEL<8>), GRID, BLOCK, LDS, ST, __VA_ARGS__); \
    else hipLaunchKernelGGL((KERNEL<16>), GRID, BLOCK, LDS, ST, __VA_ARGS__);              \
  } while (0)

// smallest power of two s with amax <= 448 s (1 for amax == 0)
__device__ __forceinline__ float pow2_scale_448(float amax) {
  if (!(amax > 0.f)) return 1.f;
  int e;
  frexpf(amax / 448.0f, &e);   // amax/448 in [2^(e-1), 2^e)
  float s = ldexpf(1.f, e);
  if (amax <= 448.0f * ldexpf(1.f, e - 1)) s = ldexpf(1.f, e - 1);
  if (amax > 448.0f * s) s *= 2.f;
  return s;
}

// ---------------------------------------------------------------------------
template <int SM>
__global__ __launch_bounds__(256) void k_qkv_finish(QkvFinishArgs a) {
  const int r = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  const int seq = a.tok0 + r;
  const int D = a.head_dim, Hq = a.n_q_heads, Hkv = a.n_kv_heads;
  const int QD = Hq * D, N = (Hq + 2 * Hkv) * D;
  if (c >= N) return;
  // the sequence's length, capacity and offset first, all together
  const int L = a.kv_len[seq];
  const int cap = a.kv_kind == KV_RING ? 0 : a.kv_cap[seq];
  const long long kv_off = a.kv_kind == KV_RING ? 0 : a.kv_off[seq];
  const int pos = L - 1;
  const bool ok = (L >= 1) && (a.kv_kind == KV_RING || L <= cap);
  if (!ok && c == 0 && a.err) atomicOr(a.err, ERR_KV_LEN);
  float v = part_sum<SM>(a.pv, r, c);
  if (a.rope_theta > 0.f && c < QD + Hkv * D) {
    // RoPE: the pair (2i, 2i+1) of the head turned by pos * theta^(-2i/D);
    // the angle and its sine and cosine in double, the rotation in fp32
    const int d = c % D, i = d >> 1;
    const float w = part_sum<SM>(a.pv, r, c ^ 1);
    const double ang = (double)pos * exp2(-(2.0 * i / D) * log2((double)a.rope_theta));
    const float cs = (float)cos(ang), sn = (float)sin(ang);
    v = (d & 1) ? w * sn + v * cs : v * cs - w * sn;
  }
  if (c < QD) {
    if (a.kv_dtype == DT_BF16) ((uint16_t*)a.q_out)[(long long)r * QD + c] = f32_to_bf16(v);
    else ((float*)a.q_out)[(long long)r * QD + c] = v;
    return;
  }
  if (!ok) return;
  const bool is_k = c < QD + Hkv * D;
  const int g = (is_k ? c - QD : c - QD - Hkv * D) / D, d = c % D;
  long long base;
  int slot;
  if (a.kv_kind == KV_RING) {
    base = ((long long)seq * Hkv + g) * a.window * D;
    slot = pos % a.window;
  } else {
    base = (kv_off * Hkv + (long long)g * cap) * D;
    slot = pos;
  }
  const long long off = is_k ? base + k_offset(slot, d, a.kv_dtype == DT_BF16 ? 32 : 16)
                             : base + (long long)(slot >> 5) * 32 * D + (long long)d * 32 + v_slot(slot & 31);
  void* cache = is_k ? a.k_cache : a.v_cache;
  if (a.kv_dtype == DT_BF16) ((uint16_t*)cache)[off] = f32_to_bf16(v);
  else ((float*)cache)[off] = v;
}

hipError_t launch_qkv_finish(const QkvFinishArgs& a, hipStream_t st) {
  const int N = (a.n_q_heads + 2 * a.n_kv_heads) * a.head_dim;
  SPA_LAUNCH_SPLITS(a.pv.S, k_qkv_finish, dim3(a.n_tok, (N + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Output projection finish of token row r by a kRowThreads workgroup (red:
// kRowThreads / 64 floats of LDS).
template <int SM>
__device__ __forceinline__ void oproj_finish_row(const OprojFinishArgs& a, int r, float* red) {
  const long long row = (long long)r * a.H;
  float h[kRowCols];
  float ss = 0.f;
  // every load of the thread first (columns past the row clamped to its
  // last), the norm weights included, then the sums
  float xv[kRowCols], yv[kRowCols], gv[kRowCols];
#pragma unroll
  for (int i = 0; i < kRowCols; ++i) {
    const int c = min(threadIdx.x + kRowThreads * i, a.H - 1);
    xv[i] = a.x[row + c];
    yv[i] = part_sum<SM>(a.pv, r, c);
    gv[i] = a.gamma[c];
  }
#pragma unroll
  for (int i = 0; i < kRowCols; ++i) {
    const int c = threadIdx.x + kRowThreads * i;
    h[i] = 0.f;
    if (c < a.H) {
      h[i] = xv[i] + yv[i];
      a.h_out[row + c] = h[i];
    }
    ss += h[i] * h[i];
  }
  ss = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(ss / (float)a.H + a.eps);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kRowCols; ++i) {
    const int c = threadIdx.x + kRowThreads * i;
    if (c < a.H) {
      h[i] = h[i] * rstd * gv[i];
      a.hn_f32[row + c] = h[i];
      if (a.hn_bf16) a.hn_bf16[row + c] = f32_to_bf16(h[i]);
      amax = fmaxf(amax, fabsf(h[i]));
    }
  }
  if (a.hn_e4m3) {
    amax = block_max(amax, red);
    const float s = pow2_scale_448(amax);
    const float inv_s = 1.0f / s;   // exact: power of two
    if (threadIdx.x == 0) a.hn_scale[r] = s;
#pragma unroll
    for (int i = 0; i < kRowCols; ++i) {
      const int c = threadIdx.x + kRowThreads * i;
      if (c < a.H) a.hn_e4m3[row + c] = f32_to_e4m3(h[i] * inv_s);
    }
  }
}

template <int SM>
__global__ __launch_bounds__(kRowThreads) void k_oproj_finish(OprojFinishArgs a) {
  __shared__ float red[kRowThreads / 64];
  oproj_finish_row<SM>(a, blockIdx.x, red);
}

hipError_t launch_oproj_finish(const OprojFinishArgs& a, hipStream_t st) {
  SPA_LAUNCH_SPLITS(a.pv.S, k_oproj_finish, dim3(a.n_tok), dim3(kRowThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router top-k of token t by one wave. Lanes hold the logits of experts
// lane + 64 j (summed over the splits in split order); k rounds of a wave
// argmax on (value, index) - larger value wins, equal values go to the lower
// index - leave the picks in pick order in pv/pi on every lane. With
// store_logits the summed logits are written to a.logits.
template <int SM>
__device__ __forceinline__ void route_token(const RouteArgs& a, int t, int lane, bool store_logits, float (&pv)[8],
                                            int (&pi)[8]) {
  const int E = a.E, k = a.k;
  float v[4];
  // every logit's split loads first (experts past E clamped to the last),
  // for the 2 or 4 experts a lane holds
  if (E <= 128) {
#pragma unroll
    for (int j = 0; j < 2; ++j) v[j] = part_sum<SM>(a.pv, t, min(lane + 64 * j, E - 1));
    v[2] = v[3] = 0.f;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = part_sum<SM>(a.pv, t, min(lane + 64 * j, E - 1));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      if (store_logits) a.logits[(long long)t * E + e] = v[j];
    } else {
      v[j] = -INFINITY;
    }
  }
  for (int p = 0; p < k; ++p) {
    float bv = v[0];
    int bi = lane;
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (v[j] > bv) {
        bv = v[j];
        bi = lane + 64 * j;
      }
    // the wave's largest (value, index), ties to the lower index: a total
    // order, so any pairing of the lanes gives the same pick (DPP inside each
    // row, lane shuffles across rows)
    auto take = [&](float ov, int oi) {
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    };
    take(__int_as_float(dpp_partner<0>(__float_as_int(bv))), dpp_partner<0>(bi));
    take(__int_as_float(dpp_partner<1>(__float_as_int(bv))), dpp_partner<1>(bi));
    take(__int_as_float(dpp_partner<2>(__float_as_int(bv))), dpp_partner<2>(bi));
    take(__int_as_float(dpp_partner<3>(__float_as_int(bv))), dpp_partner<3>(bi));
    take(__shfl_xor(bv, 16, 64), __shfl_xor(bi, 16, 64));
    take(__shfl_xor(bv, 32, 64), __shfl_xor(bi, 32, 64));
    pv[p] = bv;
    pi[p] = bi;
    if ((bi & 63) == lane) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == (bi >> 6)) v[j] = -INFINITY;
    }
  }
}

// The picks of token t and their softmax weights (lane 0 writes). AGENT:
// the picks are stored at agent scope, through to where the XCDs' caches
// agree, for a workgroup of the same launch to read.
template <bool AGENT = false>
__device__ __forceinline__ void store_picks(const RouteArgs& a, int t, int lane, const float (&pv)[8],
                                            const int (&pi)[8]) {
  if (lane != 0) return;
  const int k = a.k;
  float den = 0.f;
  for (int p = 0; p < k; ++p) den += __expf(pv[p] - pv[0]);
  for (int p = 0; p < k; ++p) {
    if constexpr (AGENT) __hip_atomic_store(a.topk_idx + t * k + p, pi[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else a.topk_idx[t * k + p] = pi[p];
    a.topk_w[t * k + p] = __expf(pv[p] - pv[0]) / den;
    if (a.topk_rec) a.topk_rec[t * k + p] = pi[p];
  }
}

// tokens per routing workgroup (one wave each)
#ifndef SPA_TOPK_TPW
#define SPA_TOPK_TPW 2
#endif
constexpr int kTopkTpw = SPA_TOPK_TPW;

// Router top-k and softmax over the picks: one wave per token.
template <int SM>
__global__ __launch_bounds__(256) void k_route_topk(RouteArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkTpw + wave;
  if (wave >= kTopkTpw || t >= a.n_tok) return;
  float pv[8];
  int pi[8];
  route_token<SM>(a, t, lane, true, pv, pi);
  store_picks(a, t, lane, pv, pi);
}

__device__ __forceinline__ void permute_body(const RouteArgs& a, char* lds, bool store);

// Top-k as above, and the permutation run by the workgroup that finishes
// last, instead of a second launch. Each wave stores its picks at agent scope
// and waits for the stores to complete; the workgroup then counts itself in
// on the arrival counter. The workgroup that takes the last count reads every
// pick at agent scope, computes the permutation and clears the counter for
// the next launch. No workgroup waits for another, and the permutation is
// the separate kernel's, bit for bit.
template <int SM>
__global__ __launch_bounds__(256) void k_route_topk_perm(RouteArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkTpw + wave;
  if (wave < kTopkTpw && t < a.n_tok) {
    float pv[8];
    int pi[8];
    route_token<SM>(a, t, lane, true, pv, pi);
    store_picks<true>(a, t, lane, pv, pi);
  }
  __builtin_amdgcn_s_waitcnt(0);   // this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  int* grp = (int*)lds;
  const int P = a.n_tok * a.k;
  for (int p = threadIdx.x; p < P; p += blockDim.x)
    grp[p] = __hip_atomic_load(a.topk_idx + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) % a.E_res;
  __syncthreads();
  permute_body(a, lds, true);
  if (threadIdx.x == 0) __hip_atomic_store(a.arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Dispatch permutation of the picks (pick p = token * k + slot runs on
// resident expert grp[p] = topk_idx[p] % E_res, grp in LDS on entry): counts,
// exclusive offsets, rows grouped by expert with (token, slot) ascending
// inside, and the inverse map; then the gather of the expert input rows. Ranks
// come from per-expert bitmasks over the picks, so no order depends on timing.
// Every workgroup computes the whole (small) permutation; the one with store
// set stores it, and the gather is dealt over the workgroups.
__device__ __forceinline__ void permute_body(const RouteArgs& a, char* lds, bool store) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int k = a.k, P = a.n_tok * k, E_res = a.E_res;
  int* grp = (int*)lds;                         // [P]
  int* rtok = grp + P;                          // [P] token of each dispatch row
  int* counts = rtok + P;                       // [E_res]
  int* offs = counts + E_res;                   // [E_res + 1]
  const int W64 = (P + 63) >> 6;
  unsigned long long* masks = (unsigned long long*)(((uintptr_t)(offs + E_res + 1) + 7) & ~(uintptr_t)7);
  for (int i = tid; i < E_res; i += nthr) counts[i] = 0;
  for (int i = tid; i < E_res * W64; i += nthr) masks[i] = 0ull;
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int g = grp[p];
    atomicAdd(&counts[g], 1);
    atomicOr(&masks[g * W64 + (p >> 6)], 1ull << (p & 63));
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int g = 0; g < E_res; ++g) {
      offs[g] = s;
      s += counts[g];
    }
    offs[E_res] = s;
  }
  __syncthreads();
  if (store)
    for (int i = tid; i <= E_res; i += nthr) a.offsets[i] = offs[i];
  for (int p = tid; p < P; p += nthr) {
    const int g = grp[p];
    const unsigned long long* mk = masks + g * W64;
    int rank = 0;
    for (int w = 0; w < (p >> 6); ++w) rank += __popcll(mk[w]);
    rank += __popcll(mk[p >> 6] & ((1ull << (p & 63)) - 1ull));
    const int row = offs[g] + rank;
    rtok[row] = p / k;
    if (store) {
      a.row_tok[row] = p / k;
      a.row_slot[row] = p % k;
      a.inv[p] = row;
    }
  }
  if (!a.gsrc) return;
  __syncthreads();
  // expert input rows in dispatch order, k-step-major: 16-byte chunk i of
  // [kstep][row][4] <- its source chunk, the chunks dealt over the workgroups
  const int ksteps = a.gK * a.gesz / 64;
  const long long total = (long long)ksteps * P * 4;
  const u32x4* src = (const u32x4*)a.gsrc;
  u32x4* dst = (u32x4*)a.gdst;
  // GU chunks per thread in flight: all loads of a round, then its stores
  constexpr int GU = 8;
  const long long stride = (long long)gridDim.x * nthr;
  for (long long i0 = (long long)blockIdx.x * nthr + tid; i0 < total; i0 += GU * stride) {
    u32x4 v[GU];
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const long long i = min(i0 + u * stride, total - 1);   // past the end: a repeat, not stored
      const long long t = i >> 2;
      v[u] = src[((long long)rtok[(int)(t % P)] * ksteps + t / P) * 4 + (i & 3)];
    }
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const long long i = i0 + u * stride;
      if (i < total) dst[i] = v[u];
    }
  }
  if (a.gdst_scale)   // one scale per dispatch row
    for (int r = blockIdx.x * nthr + tid; r < P; r += (int)stride) a.gdst_scale[r] = a.gsrc_scale[rtok[r]];
}

__global__ __launch_bounds__(256) void k_route_permute(RouteArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int* grp = (int*)lds;
  const int P = a.n_tok * a.k;
  for (int p = threadIdx.x; p < P; p += blockDim.x) grp[p] = a.topk_idx[p] % a.E_res;
  __syncthreads();
  permute_body(a, lds, blockIdx.x == 0);
}

int route_lds_bytes(int n_tok, int k, int E_res) {
  const int P = n_tok * k;
  return (2 * P + 2 * E_res + 1) * 4 + 16 + E_res * ((P + 63) / 64) * 8;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  (void)init_kernel_attributes();
  int wgs = 1;
  if (a.gsrc) {   // enough workgroups for the gather: ~8 chunks per thread, at most 64
    const long long chunks = (long long)a.gK * a.gesz / 16 * a.n_tok * a.k;
    wgs = (int)std::min<long long>(64, std::max<long long>(1, chunks / (256 * 8)));
  }
  const int lds = route_lds_bytes(a.n_tok, a.k, a.E_res);
  if (a.arrive && !a.gsrc) {   // one launch: the last top-k workgroup permutes
    SPA_LAUNCH_SPLITS(a.pv.S, k_route_topk_perm, dim3((a.n_tok + kTopkTpw - 1) / kTopkTpw), dim3(256), lds, st, a);
    return hipGetLastError();
  }
  SPA_LAUNCH_SPLITS(a.pv.S, k_route_topk, dim3((a.n_tok + kTopkTpw - 1) / kTopkTpw), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_route_permute, dim3(wgs), dim3(256), lds, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The MoE head as one persistent launch: a stage worker whose G resident
// workgroups (kRowThreads threads each, G at most one per CU of the stream's
// pool, so all are resident at once) run four phases with device hand-offs
// between them, instead of four dependent launches:
//   0. output projection finish (h, hn and the expert input rows), token rows
//      dealt over the workgroups;
//   1. router GEMV tiles: the tiles of the router product, four 256-thread
//      groups of a workgroup each running one (the same tile arithmetic as
//      the separate router launch), in lockstep;
//   2. router top-k and softmax, one wave per token;
//   3. dispatch permutation and gather of the expert input rows (every
//      workgroup computes the permutation, workgroup 0 stores it, the gather
//      is dealt over the workgroups).
// Every phase reuses the separate kernels' device code, so the results are
// those of the separate launches bit for bit, whatever G is. Hand-off: each
// workgroup finishes its stores, releases them at agent scope (the L2s of
// the XCDs are not coherent with each other) and adds one to an arrival
// counter; it then polls the counter (relaxed) until every workgroup of the
// phase has arrived and acquires at agent scope. The polls are bounded: past
// the limit the kernel sets the error bit and goes on rather than waiting
// forever. The last workgroup to leave clears the counters for the next
// launch.
constexpr unsigned kHeadSpinLimit = 1u << 22;

__device__ __forceinline__ void head_barrier(unsigned* ctr, unsigned target, int* err) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++spins > kHeadSpinLimit) {
        atomicOr(err, ERR_HANDOFF);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

template <int MT>
__device__ __forceinline__ void gemm_tile_idle() {   // the barriers of one gemm_tile<.., MT> call
#pragma unroll
  for (int i = 0; i < gemm_tile_barriers<1, MT>(); ++i) __syncthreads();
}

template <int SM0, int SM2, int MT>
__global__ __launch_bounds__(kRowThreads) void k_moe_head(MoeHeadArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const unsigned G = gridDim.x;
  // 0: output projection finish
  for (int r = blockIdx.x; r < a.of.n_tok; r += G) oproj_finish_row<SM0>(a.of, r, (float*)lds);
  head_barrier(a.ctr, G, a.err);
  // 1: router product tiles, four 256-thread groups per workgroup
  {
    const int grp = threadIdx.x >> 8, tid = threadIdx.x & 255;
    char* red = lds + grp * gemm_red_bytes<1, MT>();
    // tile t0 + grp * G + blockIdx.x: spread over the workgroups first
    for (int t0 = 0; t0 < a.n_router_tiles; t0 += 4 * (int)G) {
      const int t = t0 + grp * (int)G + blockIdx.x;
      if (t < a.n_router_tiles) gemm_tile<DT_F32, EPI_PARTIAL, 1, MT, 2>(a.router, t, tid, red);   // 2-deep ring: 1024-thread register budget
      else gemm_tile_idle<MT>();
    }
  }
  head_barrier(a.ctr, 2 * G, a.err);
  // 2: top-k and softmax weights, one wave per token
  {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int t = blockIdx.x * (kRowThreads / 64) + wave; t < a.ra.n_tok; t += G * (kRowThreads / 64)) {
      float pv[8];
      int pi[8];
      route_token<SM2>(a.ra, t, lane, true, pv, pi);
      store_picks(a.ra, t, lane, pv, pi);
    }
  }
  head_barrier(a.ctr, 3 * G, a.err);
  // 3: permutation and gather
  {
    int* grp = (int*)lds;
    const int P = a.ra.n_tok * a.ra.k;
    for (int p = threadIdx.x; p < P; p += blockDim.x) grp[p] = a.ra.topk_idx[p] % a.ra.E_res;
    __syncthreads();
    permute_body(a.ra, lds, blockIdx.x == 0);
  }
  // the last workgroup out clears the counters (every workgroup is past its polls)
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == G - 1) {
      __hip_atomic_store(a.ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ctr + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

int moe_head_lds_bytes(int n_tok, int k, int E_res) {
  return std::max({4 * gemm_red_bytes<1, 4>(), route_lds_bytes(n_tok, k, E_res), (int)(kRowThreads / 64 * sizeof(float))});
}

template <int SM0, int MT>
static hipError_t launch_head_t(const MoeHeadArgs& a, int G, int lds, hipStream_t st) {
  hipLaunchKernelGGL((k_moe_head<SM0, 16, MT>), dim3(G), dim3(kRowThreads), lds, st, a);
  return hipGetLastError();
}

bool moe_head_supported(int oproj_splits, int router_splits, int router_blk_rows) {
  return oproj_splits > 2 && oproj_splits <= 16 && router_splits > 8 && router_splits <= 16 &&
         (router_blk_rows == 16 || router_blk_rows == 32 || router_blk_rows == 64);
}

hipError_t launch_moe_head(const MoeHeadArgs& a, int G, hipStream_t st) {
  if (!moe_head_supported(a.of.pv.S, a.ra.pv.S, a.router.blk_rows) || G < 1) return hipErrorInvalidValue;
  const int lds = moe_head_lds_bytes(a.ra.n_tok, a.ra.k, a.ra.E_res);
  const int S0 = a.of.pv.S;
#define SPA_HEAD(SMV)                                                      \
  switch (a.router.blk_rows) {                                             \
    case 16: return launch_head_t<SMV, 1>(a, G, lds, st);                 \
    case 32: return launch_head_t<SMV, 2>(a, G, lds, st);                 \
    default: return launch_head_t<SMV, 4>(a, G, lds, st);                 \
  }
  if (S0 <= 4) { SPA_HEAD(4) }
  if (S0 <= 8) { SPA_HEAD(8) }
  SPA_HEAD(16)
#undef SPA_HEAD
}

// Kernel attributes set once per process before any launch (not inside a
// stream capture): the permutation may need more than the default 64 KB of LDS.
hipError_t init_kernel_attributes() {
  static hipError_t e = [] {
    hipError_t r = hipFuncSetAttribute((const void*)k_route_permute, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    for (const void* f : {(const void*)k_moe_head<4, 16, 1>, (const void*)k_moe_head<4, 16, 2>,
                          (const void*)k_moe_head<4, 16, 4>, (const void*)k_moe_head<8, 16, 1>,
                          (const void*)k_moe_head<8, 16, 2>, (const void*)k_moe_head<8, 16, 4>,
                          (const void*)k_moe_head<16, 16, 1>, (const void*)k_moe_head<16, 16, 2>,
                          (const void*)k_moe_head<16, 16, 4>})
      if (r == hipSuccess) r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    for (const void* f : {(const void*)k_route_topk_perm<1>, (const void*)k_route_topk_perm<2>,
                          (const void*)k_route_topk_perm<4>, (const void*)k_route_topk_perm<8>,
                          (const void*)k_route_topk_perm<16>})   // beside a little static LDS; the
      // permutation needs at most ~100 KB (4096 picks, 128 resident experts)
      if (r == hipSuccess) r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    return r;
  }();
  return e;
}

// ---------------------------------------------------------------------------
template <int SM>
__device__ __forceinline__ float y_elem(const CombineArgs& a, int row, int c) {
  return a.y ? a.y[(long long)row * a.H + c] : part_sum<SM>(a.ypv, row, c);
}

template <int SM>
__global__ __launch_bounds__(kRowThreads) void k_combine(CombineArgs a) {
  __shared__ float red[kRowThreads / 64];
  __shared__ float s_w[8];
  __shared__ int s_row[8];
  const int t = blockIdx.x;
  const long long row = (long long)t * a.H;
  // the residual row and the next norm's weights do not depend on the picks:
  // loaded with them, ahead of the barrier (columns past the row clamped)
  float hv[kRowCols], gv[kRowCols];
#pragma unroll
  for (int i = 0; i < kRowCols; ++i) {
    const int c = min(threadIdx.x + kRowThreads * i, a.H - 1);
    hv[i] = a.h[row + c];
    gv[i] = a.gamma_next ? a.gamma_next[c] : 0.f;
  }
  if (threadIdx.x < a.k) {
    const int r = a.inv[t * a.k + threadIdx.x];
    s_w[threadIdx.x] = a.w[t * a.k + threadIdx.x];
    s_row[threadIdx.x] = r;
  }
  __syncthreads();
  float v[kRowCols];
  float ss = 0.f;
  const int k = a.k;
  // x = h + sum over the picks in pick order of w * y. With up to 4 picks
  // and 4 splits all of the thread's loads are issued before the first add
  // (a clamped pick stands in for a missing one); the sums are the same.
  constexpr int KB = 4;
  float yv[kRowCols][KB];
  const bool batched = SM <= 4 && k >= 1 && k <= KB;
  if (batched) {
    // plain expert rows are a product of one split: no branch between loads
    const PartView pv = a.y ? PartView{a.y, 1, 0, a.H} : a.ypv;
#pragma unroll
    for (int i = 0; i < kRowCols; ++i) {
      const int c = min(threadIdx.x + kRowThreads * i, a.H - 1);
#pragma unroll
      for (int s = 0; s < KB; ++s) yv[i][s] = part_sum<SM>(pv, s_row[min(s, k - 1)], c);
    }
  }
#pragma unroll
  for (int i = 0; i < kRowCols; ++i) {
    const int c = threadIdx.x + kRowThreads * i;
    v[i] = 0.f;
    if (c < a.H) {
      float x = hv[i];
      if (batched) {
#pragma unroll
        for (int s = 0; s < KB; ++s)
          if (s < k) x += s_w[s] * yv[i][s];
      } else {
        for (int s = 0; s < k; ++s) x += s_w[s] * y_elem<SM>(a, s_row[s], c);
      }
      v[i] = x;
      a.x_out[row + c] = x;
    }
    ss += v[i] * v[i];
  }
  if (!a.gamma_next) return;
  ss = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(ss / (float)a.H + a.eps);
#pragma unroll
  for (int i = 0; i < kRowCols; ++i) {
    const int c = threadIdx.x + kRowThreads * i;
    if (c < a.H) {
      const float xn = v[i] * rstd * gv[i];
      const int ks = a.xn_dtype == DT_BF16 ? 32 : 16;   // elements per 64-byte k-step
      const long long xi = a.xn_kmajor_rows > 0 ? ((long long)(c / ks) * a.xn_kmajor_rows + t) * ks + c % ks : row + c;
      if (a.xn_dtype == DT_BF16) ((uint16_t*)a.xn_out)[xi] = f32_to_bf16(xn);
      else ((float*)a.xn_out)[xi] = xn;
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  SPA_LAUNCH_SPLITS(a.y ? 1 : a.ypv.S, k_combine, dim3(a.n_tok), dim3(kRowThreads), 0, st, a);
  return hipGetLastError();
}

// Rows of a grouped split product summed over the splits: out[r][c] for
// dispatch rows r (grouped by expert through group offsets).
template <int SM>
__global__ __launch_bounds__(256) void k_part_rows(CombineArgs a) {
  const int r = blockIdx.x;
  if (r >= a.y_group_off[a.y_n_groups]) return;
  for (int c = threadIdx.x; c < a.H; c += 256) a.x_out[(long long)r * a.H + c] = y_elem<SM>(a, r, c);
}

hipError_t launch_part_rows(const CombineArgs& a, int max_rows, hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  SPA_LAUNCH_SPLITS(a.y ? 1 : a.ypv.S, k_part_rows, dim3(max_rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row conversion, one workgroup of T threads per row: rows of up to 4,096
// columns are read once into registers (4,096 / T per thread, every load
// issued before the first use), the row's largest magnitude is a block
// reduction, then the codes are written; longer rows read their columns again
// for the second pass. Thread t holds columns t + T j. Few rows take T = 1,024
// (more waves per row while the rows leave CUs idle), many rows T = 256.
constexpr int kCvtRowCols = 4096;   // longest row held in registers

template <int T>
__global__ __launch_bounds__(T) void k_cvt_rows(CvtArgs a) {
  constexpr int kRegCols = kCvtRowCols / T;
  __shared__ float red[T / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const long long R = a.kmajor_rows;
  // element c of row r: row-major, or k-step-major with 16 fp32 per k-step
  auto in_idx = [&](int c) -> long long {
    return R ? ((long long)(c >> 4) * R + r) * 16 + (c & 15) : (long long)r * a.n_cols + c;
  };
  const bool e4m3 = a.dtype != DT_BF16;
  // output c: bf16 (32 per k-step) or E4M3 (64 per k-step)
  auto store = [&](int c, float x, float inv_s) {
    if (!e4m3) {
      const long long o = R ? ((long long)(c >> 5) * R + r) * 32 + (c & 31) : (long long)r * a.n_cols + c;
      ((uint16_t*)a.out)[o] = f32_to_bf16(x);
    } else {
      const long long o = R ? ((long long)(c >> 6) * R + r) * 64 + (c & 63) : (long long)r * a.n_cols + c;
      ((uint8_t*)a.out)[o] = f32_to_e4m3(x * inv_s);
    }
  };
  // the row's scale from this thread's largest magnitude (E4M3)
  auto row_scale = [&](float amax) {
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int w = 1; w < T / 64; ++w) m = fmaxf(m, red[w]);
    const float s = pow2_scale_448(m);
    if (tid == 0) a.scales[r] = s;
    return 1.0f / s;   // exact: power of two
  };
  if (a.n_cols <= kCvtRowCols) {
    float v[kRegCols];
#pragma unroll
    for (int j = 0; j < kRegCols; ++j) {
      const int c = tid + T * j;
      const float x = a.x[in_idx(min(c, a.n_cols - 1))];   // clamped: no branch between the loads
      v[j] = c < a.n_cols ? x : 0.f;
    }
    float inv_s = 1.f;
    if (e4m3) {
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < kRegCols; ++j) amax = fmaxf(amax, fabsf(v[j]));
      inv_s = row_scale(amax);
    }
#pragma unroll
    for (int j = 0; j < kRegCols; ++j) {
      const int c = tid + T * j;
      if (c < a.n_cols) store(c, v[j], inv_s);
    }
    return;
  }
  float inv_s = 1.f;
  if (e4m3) {
    float amax = 0.f;
    for (int c = tid; c < a.n_cols; c += T) amax = fmaxf(amax, fabsf(a.x[in_idx(c)]));
    inv_s = row_scale(amax);
  }
  for (int c = tid; c < a.n_cols; c += T) store(c, a.x[in_idx(c)], inv_s);
}

hipError_t launch_cvt_rows(const CvtArgs& a, hipStream_t st) {
  if (a.n_rows <= 0 || a.n_cols <= 0) return hipSuccess;
  if (a.n_rows >= 2 * a.n_cus) hipLaunchKernelGGL(k_cvt_rows<256>, dim3(a.n_rows), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_cvt_rows<1024>, dim3(a.n_rows), dim3(1024), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 16-byte chunk i of the panel layout <- its source chunk (or zero past row N).
__global__ void k_pack_panels(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int N, int ksteps, int n_panels,
                              long long total) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int q = (int)(i & 3);                      // 16-byte quarter of the 64-byte k-step
    const int row16 = (int)((i >> 2) & 15);
    long long t = i >> 6;                            // (mat, panel, kstep)
    const int ks = (int)(t % ksteps);
    t /= ksteps;
    const int panel = (int)(t % n_panels);
    const long long mat = t / n_panels;
    const int n = panel * 16 + row16;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < N) v = src[((mat * N + n) * ksteps + ks) * 4 + q];
    dst[i] = v;
  }
}

hipError_t launch_pack_panels(const void* src, void* dst, int n_mats, int N, int K, int esz, hipStream_t st) {
  const int ksteps = K * esz / 64, n_panels = (N + 15) / 16;
  const long long total = (long long)n_mats * n_panels * ksteps * 64;
  if (total <= 0) return hipSuccess;
  long long g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_pack_panels, dim3((int)g), dim3(256), 0, st, (const u32x4*)src, (u32x4*)dst, N, ksteps, n_panels,
                     total);
  return hipGetLastError();
}

// 16-byte chunk i of the k-step-major destination [kstep][r][4 quarters].
__global__ void k_gather_kmajor(const u32x4* __restrict__ src, const int* __restrict__ row_src, int R, int ksteps,
                                u32x4* __restrict__ dst, const float* __restrict__ src_scale, float* __restrict__ dst_scale) {
  const long long total = (long long)ksteps * R * 4;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int q = (int)(i & 3);
    const long long t = i >> 2;
    const int r = (int)(t % R);
    const int ks = (int)(t / R);
    const long long srow = row_src[r];
    dst[i] = src[(srow * ksteps + ks) * 4 + q];
    if (dst_scale && ks == 0 && q == 0) dst_scale[r] = src_scale[srow];
  }
}

hipError_t launch_gather_kmajor(const void* src, const int* row_src, int R, int K, int esz, void* dst,
                                const float* src_scale, float* dst_scale, hipStream_t st) {
  const int ksteps = K * esz / 64;
  const long long total = (long long)ksteps * R * 4;
  if (total <= 0) return hipSuccess;
  long long g = (total + 255) / 256;
  if (g > 8192) g = 8192;
  hipLaunchKernelGGL(k_gather_kmajor, dim3((int)g), dim3(256), 0, st, (const u32x4*)src, row_src, R, ksteps,
                     (u32x4*)dst, src_scale, dst_scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ void k_fill_i32(int* p, long long n, int v) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ __launch_bounds__(64) void k_span_fold(unsigned long long* spans, int n, unsigned long long* acc) {
  if (threadIdx.x != 0) return;
  unsigned long long sum = 0, cnt = 0;
  for (int i = 0; i < n; ++i) {
    unsigned long long* w = spans + (long long)i * kSpanWords;
    unsigned long long end = 0;
    for (int j = 1; j <= 16; ++j) end = w[8 * j] > end ? w[8 * j] : end;
    if (w[0] != 0 && end >= w[0]) {   // else a launch that did no timed work
      sum += end - w[0];
      cnt += 1;
    }
    w[0] = 0;   // cleared for the next iteration's launches
    for (int j = 1; j <= 16; ++j) w[8 * j] = 0;
  }
  acc[0] += sum;
  acc[1] += cnt;
}

hipError_t launch_span_fold(unsigned long long* spans, int n, unsigned long long* acc, hipStream_t st) {
  hipLaunchKernelGGL(k_span_fold, dim3(1), dim3(64), 0, st, spans, n, acc);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, long long n, int v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(k_fill_i32, dim3((int)g), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// Virtual communication endpoint. The copy stands for the endpoint's local
// traffic (send buffer read, receive buffer written); the wait makes the
// launch last the collective's modelled time. Wave 0 of each workgroup polls
// the wall clock with short sleeps; the iteration cap (each iteration sleeps
// for more than one clock tick) ends the wait even if the clock stalled.
__global__ __launch_bounds__(256) void k_virtual_comm(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                      long long n16, unsigned long long ticks) {
  const unsigned long long t0 = wall_clock64();
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (long long)gridDim.x * blockDim.x)
    dst[i] = src[i];
  if (threadIdx.x < 64) {
    const unsigned long long cap = ticks + 1024;
    for (unsigned long long it = 0; it < cap && wall_clock64() - t0 < ticks; ++it) __builtin_amdgcn_s_sleep(2);
  }
  __syncthreads();
}

hipError_t launch_virtual_comm(const void* src, void* dst, long long n16, unsigned long long ticks, hipStream_t st) {
  long long g = (n16 + 2047) / 2048;   // 32 KB per workgroup
  g = g < 1 ? 1 : (g > 128 ? 128 : g);
  hipLaunchKernelGGL(k_virtual_comm, dim3((int)g), dim3(256), 0, st, (const u32x4*)src, (u32x4*)dst, n16, ticks);
  return hipGetLastError();
}

// KV cache rows <-> [n][Hkv][D] (one (sequence, position) per row, all KV heads).
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
      if (pos >= a.kv_cap[seq]) continue;
      base = (a.kv_off[seq] * a.n_kv_heads + (long long)g * a.kv_cap[seq]) * D;
      slot = pos;
    }
    const long long ko = base + k_offset(slot, d, a.kv_dtype == DT_BF16 ? 32 : 16);
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
  const unsigned xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11));   // HW_REG_XCC_ID
  const unsigned hw = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));     // HW_REG_HW_ID
  const long long t0 = clock64();
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
