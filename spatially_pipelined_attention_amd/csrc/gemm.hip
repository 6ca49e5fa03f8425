// Skinny matrix products of the decode layer on gfx950 MFMA.
//
// Every projection of the layer (Figure 3 of the SubGPU Pipelining paper:
// Q/KV projection, output projection, router gating, expert up, expert down)
// is Y[r][n] = sum_k X[r][k] * W[n][k] with few rows r (the decoded tokens of
// one microbatch, or the rows routed to one expert) and a large weight W that
// is read once from HBM. The kernel is built around that:
//   * a workgroup of 4 waves owns 64 output columns (16 per wave) and loops
//     over row blocks of 64; each lane streams 16 bytes of its W row per
//     k-step straight from HBM into registers, 8 k-steps ahead;
//   * X (tiny, L2-resident) is staged through LDS in 4-k-step chunks,
//     double-buffered, and shared by the 4 waves; the producer can gather
//     rows and apply RMSNorm on the fly from row sum-of-squares partials;
//   * the k dimension may be split over S workgroups; partial tiles meet in
//     workspace and the last workgroup to arrive (integer counter) sums them
//     in split order, so results never depend on timing;
//   * the epilogue runs on the finished 64x64 tile in LDS: q store + KV cache
//     append, residual add + row sum-of-squares, SwiGLU, plain store, or
//     router logits followed by top-k and the token->expert permutation.
// MFMA operand layout: A = W tile (16 output columns x k), B = X^T tile
// (k x 16 rows); the k order inside a k-step is the natural one.
#include "common.h"
#include "kernels.h"

namespace spa {

// bytes of one k-step of one row (16 B per lane x 4 lane groups)
constexpr int kStepBytes = 64;
constexpr int kChunkSteps = 4;                      // k-steps per LDS chunk
constexpr int kChunkBytes = kStepBytes * kChunkSteps;
constexpr int kRowPitch = kChunkBytes + 16;         // LDS row pitch (bank spread)
constexpr int kBufBytes = 64 * kRowPitch;
constexpr int kPF = 8;                              // W prefetch depth (k-steps)
constexpr int kTilePitch = 68;                      // fp32 epilogue tile pitch
constexpr int kGemmLds = 2 * kBufBytes + 64 * 4 + 64;  // X buffers + rstd + flags

template <int WT> struct WTraits;
template <> struct WTraits<DT_BF16> { static constexpr int ks = 32; static constexpr int esz = 2; };
template <> struct WTraits<DT_F32> { static constexpr int ks = 16; static constexpr int esz = 4; };
template <> struct WTraits<DT_E4M3> { static constexpr int ks = 64; static constexpr int esz = 1; };

template <int WT>
__device__ __forceinline__ f32x4 mma_step(u32x4 w, u32x4 x, f32x4 acc) {
  if constexpr (WT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(w), bitcast<bf16x8>(x), acc, 0, 0, 0);
  } else if constexpr (WT == DT_F32) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w[u]), __uint_as_float(x[u]), acc, 0, 0, 0);
    return acc;
  } else {
    long w0 = (long)((uint64_t)w[0] | ((uint64_t)w[1] << 32));
    long w1 = (long)((uint64_t)w[2] | ((uint64_t)w[3] << 32));
    long x0 = (long)((uint64_t)x[0] | ((uint64_t)x[1] << 32));
    long x1 = (long)((uint64_t)x[2] | ((uint64_t)x[3] << 32));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(w0, x0, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(w1, x1, acc, 0, 0, 0);
  }
}

// W row feeding tile column c (0..63) of column tile nb.
template <int EPI>
__device__ __forceinline__ int w_row_of(const GemmArgs& a, int nb, int c) {
  if constexpr (EPI == EPI_SWIGLU) {
    return c < 32 ? nb * 32 + c : a.inter + nb * 32 + (c - 32);
  } else {
    return nb * 64 + c;
  }
}

template <int EPI>
__device__ __forceinline__ int w_rows_total(const GemmArgs& a) {
  if constexpr (EPI == EPI_SWIGLU) return 2 * a.inter;
  else return a.N;
}

// ---------------------------------------------------------------------------
// X staging: thread t fills LDS row t/4, bytes [64*(t%4), +64) of the chunk
// row, which is exactly k-step (t%4) of the chunk for that row.
// ---------------------------------------------------------------------------
template <int WT, int XM>
struct Stager {
  static constexpr int kLoads = (XM == XM_NORM && WT == DT_BF16) ? 8 : 4;
  u32x4 v[kLoads];
  bool live;

  __device__ __forceinline__ void load(const GemmArgs& a, const int* xrow_l, int rows_here, int m,
                                       int kstep, int ks_end) {
    live = (m < rows_here) && (kstep < ks_end);
    if (!live) return;
    const int ks = WTraits<WT>::ks;
    const long long xrow = xrow_l[m];
    if constexpr (XM == XM_RAW) {
      const char* src = (const char*)a.X + (xrow * a.x_ld + (long long)kstep * ks) * WTraits<WT>::esz;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ld16(src + 16 * i);
    } else {
      const char* src = (const char*)a.X + (xrow * a.x_ld + (long long)kstep * ks) * 4;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) v[i] = ld16(src + 16 * i);
    }
  }

  __device__ __forceinline__ void store(const GemmArgs& a, char* buf, const float* rstd, int m, int part,
                                        int kstep) {
    char* dst = buf + m * kRowPitch + part * kStepBytes;
    if (!live) {
      u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) st16(dst + 16 * i, z);
      return;
    }
    if constexpr (XM == XM_RAW) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st16(dst + 16 * i, v[i]);
    } else {
      const int ks = WTraits<WT>::ks;
      const float r = rstd[m];
      const float* g = a.gamma + (long long)kstep * ks;
      if constexpr (WT == DT_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 o;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 s = v[2 * i + h];
            f32x4 gg = *reinterpret_cast<const f32x4*>(g + 8 * i + 4 * h);
            o[2 * h + 0] = pack_bf16x2(__uint_as_float(s[0]) * r * gg[0], __uint_as_float(s[1]) * r * gg[1]);
            o[2 * h + 1] = pack_bf16x2(__uint_as_float(s[2]) * r * gg[2], __uint_as_float(s[3]) * r * gg[3]);
          }
          st16(dst + 16 * i, o);
        }
      } else {  // fp32 MFMA input
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 s = v[i], o;
          f32x4 gg = *reinterpret_cast<const f32x4*>(g + 4 * i);
#pragma unroll
          for (int u = 0; u < 4; ++u) o[u] = __float_as_uint(__uint_as_float(s[u]) * r * gg[u]);
          st16(dst + 16 * i, o);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// routing tail: top-k per token, softmax over the picks, permutation
// ---------------------------------------------------------------------------
__device__ void route_tail(const GemmArgs& a, int n_tok, char* lds) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = a.N, k = a.top_k, P = n_tok * k;
  const int E_res = a.n_resident;
  const float* logits = (const float*)a.out;
  int* grp = (int*)lds;                                   // [P]
  int* counts = grp + P;                                  // [E_res]
  int* offs = counts + E_res;                             // [E_res + 1]
  const int W64 = (P + 63) >> 6;
  unsigned long long* masks = (unsigned long long*)(((uintptr_t)(offs + E_res + 1) + 7) & ~(uintptr_t)7);

  for (int t = wave; t < n_tok; t += 4) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = lane + 64 * j;
      v[j] = e < E ? logits[(long long)t * a.out_ld + e] : -INFINITY;
    }
    float pick_v[8];
    int pick_i[8];
    for (int p = 0; p < k; ++p) {
      float bv = v[0];
      int bi = lane;
#pragma unroll
      for (int j = 1; j < 4; ++j)
        if (v[j] > bv) { bv = v[j]; bi = lane + 64 * j; }   // strict: lower index wins ties
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      pick_v[p] = bv;
      pick_i[p] = bi;
      if ((bi & 63) == lane) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j == (bi >> 6)) v[j] = -INFINITY;
      }
    }
    if (lane == 0) {
      float den = 0.f;
      for (int p = 0; p < k; ++p) den += __expf(pick_v[p] - pick_v[0]);
      for (int p = 0; p < k; ++p) {
        int idx = pick_i[p];
        a.topk_idx[t * k + p] = idx;
        a.topk_w[t * k + p] = __expf(pick_v[p] - pick_v[0]) / den;
        if (a.topk_rec) a.topk_rec[t * k + p] = idx;
        grp[t * k + p] = idx % E_res;
      }
    }
  }
  for (int i = tid; i < E_res; i += 256) counts[i] = 0;
  for (int i = tid; i < E_res * W64; i += 256) masks[i] = 0ull;
  __syncthreads();
  for (int p = tid; p < P; p += 256) {
    int g = grp[p];
    atomicAdd(&counts[g], 1);
    atomicOr(&masks[g * W64 + (p >> 6)], 1ull << (p & 63));
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int g = 0; g < E_res; ++g) { offs[g] = s; s += counts[g]; }
    offs[E_res] = s;
  }
  __syncthreads();
  for (int i = tid; i <= E_res; i += 256) a.route_off[i] = offs[i];
  for (int p = tid; p < P; p += 256) {
    int g = grp[p];
    const unsigned long long* mk = masks + g * W64;
    int rank = 0;
    for (int w = 0; w < (p >> 6); ++w) rank += __popcll(mk[w]);
    rank += __popcll(mk[p >> 6] & ((1ull << (p & 63)) - 1ull));
    int row = offs[g] + rank;
    a.row_tok[row] = p / k;
    a.row_slot[row] = p % k;
    a.inv[p] = row;
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int WT, int XM, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* xbuf0 = lds;
  char* xbuf1 = lds + kBufBytes;
  float* rstd = (float*)(lds + 2 * kBufBytes);
  int* flag = (int*)(lds + 2 * kBufBytes + 64 * 4);
  __shared__ int xrow_l[64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int bid = blockIdx.x;
  const int s = bid % a.S;
  bid /= a.S;
  const int nb = bid % a.n_tiles;
  const int grp = bid / a.n_tiles;

  int r0 = 0, nrows = a.n_rows;
  if (a.group_off) {
    r0 = a.group_off[grp];
    nrows = a.group_off[grp + 1] - r0;
  }
  if (nrows <= 0) return;

  constexpr int KS = WTraits<WT>::ks;
  const int nks_total = a.K / KS;
  const int ks0 = (int)((long long)s * nks_total / a.S);
  const int ks1 = (int)((long long)(s + 1) * nks_total / a.S);
  const int nks = ks1 - ks0;

  // this lane's W row
  const int c_lane = wave * 16 + (lane & 15);
  const int wrow = w_row_of<EPI>(a, nb, c_lane);
  const bool wvalid = wrow < w_rows_total<EPI>(a);
  const char* wp = (const char*)a.W +
                   ((long long)grp * a.w_gstride + (long long)(wvalid ? wrow : 0) * a.K) * WTraits<WT>::esz +
                   (long long)ks0 * kStepBytes + (lane >> 4) * 16;

  const int n_rb = (nrows + 63) >> 6;
  for (int rb = 0; rb < n_rb; ++rb) {
    const int rows_here = min(64, nrows - rb * 64);
    const int mtiles = (rows_here + 15) >> 4;

    if (tid < 64) {
      int orow = r0 + rb * 64 + tid;
      int xr = tid < rows_here ? (a.row_src ? a.row_src[orow] : orow) : 0;
      xrow_l[tid] = xr;
      if constexpr (XM == XM_NORM) {
        float ssum = 0.f;
        if (tid < rows_here)
          for (int t = 0; t < a.ss_tiles; ++t) ssum += a.ss[(long long)t * a.ss_ld + xr];
        rstd[tid] = 1.0f / sqrtf(ssum * a.inv_h + a.eps);
      }
    }
    __syncthreads();

    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 wring[kPF];
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      wring[i] = u32x4{0u, 0u, 0u, 0u};
      if (wvalid && i < nks) wring[i] = ld16(wp + (long long)i * kStepBytes);
    }

    const int m_st = tid >> 2, part = tid & 3;
    Stager<WT, XM> st;
    const int nch = (nks + kChunkSteps - 1) / kChunkSteps;
    st.load(a, xrow_l, rows_here, m_st, ks0 + part, ks1);
    st.store(a, xbuf0, rstd, m_st, part, ks0 + part);
    lds_barrier();

    for (int c = 0; c < nch; c += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cc = c + h;
        if (cc < nch) {
          char* cur = (cc & 1) ? xbuf1 : xbuf0;
          char* nxt = (cc & 1) ? xbuf0 : xbuf1;
          const bool more = cc + 1 < nch;
          const int kstep_next = ks0 + (cc + 1) * kChunkSteps + part;
          if (more) st.load(a, xrow_l, rows_here, m_st, kstep_next, ks1);
#pragma unroll
          for (int j = 0; j < kChunkSteps; ++j) {
            const int kk = cc * kChunkSteps + j;
            if (kk < nks) {
              u32x4 wf = wring[h * kChunkSteps + j];
              if (wvalid && kk + kPF < nks) wring[h * kChunkSteps + j] = ld16(wp + (long long)(kk + kPF) * kStepBytes);
              const char* xb = cur + (lane & 15) * kRowPitch + j * kStepBytes + (lane >> 4) * 16;
#pragma unroll
              for (int mt = 0; mt < 4; ++mt)
                if (mt < mtiles) acc[mt] = mma_step<WT>(wf, ld16(xb + mt * 16 * kRowPitch), acc[mt]);
            }
          }
          if (more) st.store(a, nxt, rstd, m_st, part, kstep_next);
          lds_barrier();
        }
      }
    }

    // ---------------- split-K meeting point ----------------
    const long long tile_id = ((long long)grp * a.n_tiles + nb) * a.rb_stride + rb;
    if (a.S > 1) {
      float* my = a.part + (tile_id * a.S + s) * 4096 + tid * 16;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) *reinterpret_cast<f32x4*>(my + 4 * mt) = acc[mt];
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        int old = atomicAdd(a.ctr + tile_id, 1);
        int last = (old == a.S - 1);
        if (last) atomicExch(a.ctr + tile_id, 0);
        flag[0] = last;
      }
      __syncthreads();
      if (!flag[0]) continue;
      __threadfence();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int ss = 0; ss < a.S; ++ss) {
        const float* p = a.part + (tile_id * a.S + ss) * 4096 + tid * 16;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4 * mt));
          acc[mt] += v;
        }
      }
    }

    // ---------------- final tile -> LDS ----------------
    float* T = (float*)lds;   // reuses the X buffers (all reads done at the last barrier)
    {
      float wsc[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (WT == DT_E4M3) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int c = wave * 16 + (lane >> 4) * 4 + r;
          int wr = w_row_of<EPI>(a, nb, c);
          wsc[r] = wr < w_rows_total<EPI>(a) ? a.w_scale[(long long)grp * a.ws_gstride + wr] : 0.f;
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int m = mt * 16 + (lane & 15);
        float xs = 1.f;
        if constexpr (WT == DT_E4M3) xs = (m < rows_here) ? a.x_scale[xrow_l[m]] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) T[m * kTilePitch + wave * 16 + (lane >> 4) * 4 + r] = acc[mt][r] * wsc[r] * xs;
      }
    }
    __syncthreads();

    // ---------------- epilogue: thread -> (row, 16 columns) ----------------
    const int m = tid >> 2, cq = (tid & 3) * 16;
    const bool rvalid = m < rows_here;
    const long long orow = r0 + rb * 64 + m;
    const float* trow = T + m * kTilePitch;

    if constexpr (EPI == EPI_STORE) {
      if (rvalid) {
        float* o = (float*)a.out + orow * a.out_ld + nb * 64 + cq;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (nb * 64 + cq + i < a.N) o[i] = trow[cq + i];
      }
    } else if constexpr (EPI == EPI_RESID_SS) {
      float ssq = 0.f;
      if (rvalid) {
        const float* rs = a.resid + orow * a.resid_ld + nb * 64 + cq;
        float* o = (float*)a.out + orow * a.out_ld + nb * 64 + cq;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          f32x4 x = *reinterpret_cast<const f32x4*>(rs + i);
          f32x4 hv;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            hv[u] = x[u] + trow[cq + i + u];
            ssq += hv[u] * hv[u];
          }
          *reinterpret_cast<f32x4*>(o + i) = hv;
        }
      }
      ssq += __shfl_xor(ssq, 1, 64);
      ssq += __shfl_xor(ssq, 2, 64);
      if (rvalid && (tid & 3) == 0) a.ss_out[(long long)nb * a.ss_out_ld + orow] = ssq;
    } else if constexpr (EPI == EPI_SWIGLU) {
      if (rvalid && cq < 32) {
        const int j0 = nb * 32 + cq;
        float z[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float g = trow[cq + i], u = trow[32 + cq + i];
          z[i] = g / (1.0f + __expf(-g)) * u;
        }
        if (a.out_dtype == DT_BF16) {
          uint16_t* o = (uint16_t*)a.out + orow * a.out_ld + j0;
#pragma unroll
          for (int i = 0; i < 16; i += 8) {
            u32x4 pk = {pack_bf16x2(z[i], z[i + 1]), pack_bf16x2(z[i + 2], z[i + 3]),
                        pack_bf16x2(z[i + 4], z[i + 5]), pack_bf16x2(z[i + 6], z[i + 7])};
            st16(o + i, pk);
          }
        } else {
          float* o = (float*)a.out + orow * a.out_ld + j0;
#pragma unroll
          for (int i = 0; i < 16; ++i) o[i] = z[i];
        }
      }
    } else if constexpr (EPI == EPI_QKV) {
      if (rvalid) {
        const int D = a.head_dim;   // == 64: the tile is one head
        const int seq = a.tok0 + (int)orow;
        if (nb < a.n_q_heads) {
          if (a.out_dtype == DT_BF16) {
            uint16_t* o = (uint16_t*)a.out + orow * a.out_ld + nb * 64 + cq;
#pragma unroll
            for (int i = 0; i < 16; i += 8) {
              u32x4 pk = {pack_bf16x2(trow[cq + i], trow[cq + i + 1]), pack_bf16x2(trow[cq + i + 2], trow[cq + i + 3]),
                          pack_bf16x2(trow[cq + i + 4], trow[cq + i + 5]), pack_bf16x2(trow[cq + i + 6], trow[cq + i + 7])};
              st16(o + i, pk);
            }
          } else {
            float* o = (float*)a.out + orow * a.out_ld + nb * 64 + cq;
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = trow[cq + i];
          }
        } else {
          const bool is_k = nb < a.n_q_heads + a.n_kv_heads;
          const int g = is_k ? nb - a.n_q_heads : nb - a.n_q_heads - a.n_kv_heads;
          const int L = a.kv_len[seq];
          const int pos = L - 1;
          long long base;   // element offset of (seq, g) region
          int slot;
          if (a.kv_kind == KV_RING) {
            base = ((long long)seq * a.n_kv_heads + g) * a.window * D;
            slot = pos % a.window;
          } else {
            base = (a.kv_off[seq] * a.n_kv_heads + (long long)g * a.kv_cap[seq]) * D;
            slot = pos;
          }
          const bool ok = (L >= 1) && (a.kv_kind == KV_RING || L <= a.kv_cap[seq]);
          if (ok) {
            if (is_k) {
              long long off = base + (long long)slot * D + cq;
              if (a.kv_dtype == DT_BF16) {
                uint16_t* o = (uint16_t*)a.k_cache + off;
#pragma unroll
                for (int i = 0; i < 16; ++i) o[i] = f32_to_bf16(trow[cq + i]);
              } else {
                float* o = (float*)a.k_cache + off;
#pragma unroll
                for (int i = 0; i < 16; ++i) o[i] = trow[cq + i];
              }
            } else {
              long long off = base + (long long)(slot >> 5) * 32 * D + v_slot(slot & 31);
              if (a.kv_dtype == DT_BF16) {
                uint16_t* o = (uint16_t*)a.v_cache + off;
#pragma unroll
                for (int i = 0; i < 16; ++i) o[(cq + i) * 32] = f32_to_bf16(trow[cq + i]);
              } else {
                float* o = (float*)a.v_cache + off;
#pragma unroll
                for (int i = 0; i < 16; ++i) o[(cq + i) * 32] = trow[cq + i];
              }
            }
          } else if (a.err && (tid & 3) == 0) {
            atomicOr(a.err, ERR_KV_LEN);
          }
        }
      }
    } else if constexpr (EPI == EPI_ROUTER) {
      if (rvalid) {
        float* o = (float*)a.out + orow * a.out_ld + nb * 64 + cq;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (nb * 64 + cq + i < a.N) o[i] = trow[cq + i];
      }
      // last finished tile of the launch routes all tokens
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        const int total = a.n_tiles * n_rb;
        int old = atomicAdd(a.done_ctr, 1);
        int last = (old == total - 1);
        if (last) atomicExch(a.done_ctr, 0);
        flag[0] = last;
      }
      __syncthreads();
      if (flag[0]) {
        __threadfence();
        route_tail(a, nrows, lds);
      }
    }
    __syncthreads();   // T (aliasing the X buffers) is free again
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int WT, int XM, int EPI>
static hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  int lds_bytes = kGemmLds;
  if (EPI == EPI_ROUTER) {
    int P = a.n_rows * a.top_k;
    int need = (P + 2 * a.n_resident + 1) * 4 + 16 + a.n_resident * ((P + 63) / 64) * 8;
    if (need > lds_bytes) lds_bytes = need;
  }
  int grid = a.n_tiles * a.n_groups * a.S;
  hipLaunchKernelGGL((k_gemm<WT, XM, EPI>), dim3(grid), dim3(256), lds_bytes, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int wt, int xm, int epi, const GemmArgs& a, hipStream_t st) {
#define SPA_CASE(W, X, E) \
  if (wt == W && xm == X && epi == E) return launch_t<W, X, E>(a, st);
  SPA_CASE(DT_BF16, XM_NORM, EPI_QKV)
  SPA_CASE(DT_F32, XM_NORM, EPI_QKV)
  SPA_CASE(DT_BF16, XM_RAW, EPI_RESID_SS)
  SPA_CASE(DT_F32, XM_RAW, EPI_RESID_SS)
  SPA_CASE(DT_F32, XM_NORM, EPI_ROUTER)
  SPA_CASE(DT_BF16, XM_NORM, EPI_SWIGLU)
  SPA_CASE(DT_F32, XM_NORM, EPI_SWIGLU)
  SPA_CASE(DT_E4M3, XM_RAW, EPI_SWIGLU)
  SPA_CASE(DT_BF16, XM_RAW, EPI_STORE)
  SPA_CASE(DT_F32, XM_RAW, EPI_STORE)
  SPA_CASE(DT_E4M3, XM_RAW, EPI_STORE)
#undef SPA_CASE
  return hipErrorInvalidValue;
}

int gemm_lds_bytes() { return kGemmLds; }

}  // namespace spa
