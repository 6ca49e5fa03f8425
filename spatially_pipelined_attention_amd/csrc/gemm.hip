// Skinny matrix products of the decode layer on gfx950 MFMA.
//
// Every projection of the layer (Figure 3 of the SubGPU Pipelining paper:
// Q/KV projection, output projection, router gating, expert up, expert down)
// is Y[r][n] = sum_k X[r][k] * W[n][k] with few rows r (the decoded tokens of
// a microbatch, or the rows routed to one expert) and a large W read once
// from HBM. The kernel is built for that:
//   * a workgroup of 4 waves owns 64 output columns (16 per wave) of one
//     64-row block; each lane streams 16 bytes of its W row per k-step
//     straight from HBM into registers;
//   * X (small, L2-resident) is staged through LDS, 8 k-steps per group,
//     double-buffered, and shared by the 4 waves (optionally gathered by a
//     row map, e.g. tokens routed to an expert);
//   * the hot loop has no data-dependent branches: k-steps beyond the range
//     are masked to zero and addresses clamped, the next group's X and W
//     loads are issued (X first) before the current group is multiplied, so
//     the W stream stays in flight across the LDS barriers;
//   * the k dimension may be split over S workgroups; each writes its fp32
//     partial tile to workspace and a row-wise finish kernel sums the splits
//     in split order (no cross-workgroup fences, fixed summation order);
//   * with S = 1 the epilogue runs here on the finished tile in LDS: SwiGLU
//     (gate and up columns paired inside the tile) or a plain store, with
//     E4M3 per-row and per-channel scales applied first.
// MFMA operand layout: A = W tile (16 output columns x k), B = X^T tile
// (k x 16 rows); lane l holds C[4(l/16)+i][l%16] = Y[row l%16][col 4(l/16)+i].
#include "common.h"
#include "kernels.h"

namespace spa {

constexpr int kStepBytes = 64;                       // one k-step of one row
constexpr int kGroup = 8;                            // k-steps per pipeline group
constexpr int kGroupBytes = kStepBytes * kGroup;     // 512
constexpr int kRowPitch = kGroupBytes + 16;          // LDS row pitch (bank spread)
constexpr int kBufBytes = 64 * kRowPitch;            // one X group buffer
constexpr int kTilePitch = 68;                       // fp32 epilogue tile pitch
constexpr int kGemmLds = 2 * kBufBytes;

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
  if constexpr (EPI == EPI_SWIGLU) return c < 32 ? nb * 32 + c : a.inter + nb * 32 + (c - 32);
  else return nb * 64 + c;
}

template <int EPI>
__device__ __forceinline__ int w_rows_total(const GemmArgs& a) {
  if constexpr (EPI == EPI_SWIGLU) return 2 * a.inter;
  else return a.N;
}

// One row block: acc[mt] += X[rows] W^T over this workgroup's k-steps.
// Thread t stages LDS row t/4, k-steps 2(t%4) and 2(t%4)+1 of a group.
template <int WT, int MT>
__device__ __forceinline__ void mainloop(const GemmArgs& a, const char* wp, bool wvalid, int ks0, int nks,
                                         const char* xsrc, char* buf0, char* buf1, f32x4 (&acc)[4]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int m_st = tid >> 2, kq = (tid & 3) * 2;
  const int ngroups = (nks + kGroup - 1) / kGroup;
  const int kl = nks - 1;                       // last local k-step (clamp target)
  u32x4 WA[kGroup], WB[kGroup], XS[8];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto xload = [&](int g) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kk = min(g * kGroup + kq + i, kl);
      const char* p = xsrc + (long long)(ks0 + kk) * kStepBytes;
#pragma unroll
      for (int u = 0; u < 4; ++u) XS[4 * i + u] = ld16(p + 16 * u);
    }
  };
  auto xstore = [&](char* buf) {
    char* dst = buf + m_st * kRowPitch + kq * kStepBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) st16(dst + 16 * i, XS[i]);
  };
  auto wload = [&](int g, u32x4 (&W)[kGroup]) {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) W[j] = ld16(wp + (long long)min(g * kGroup + j, kl) * kStepBytes);
  };
  auto compute = [&](int g, const u32x4 (&W)[kGroup], const char* buf) {
    const char* xb = buf + (lane & 15) * kRowPitch + (lane >> 4) * 16;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const bool live = wvalid && (g * kGroup + j < nks);
      const u32x4 wf = live ? W[j] : zero;
      u32x4 xf[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xf[mt] = ld16(xb + mt * 16 * kRowPitch + j * kStepBytes);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mma_step<WT>(wf, xf[mt], acc[mt]);
      // keep the fragment reads of one k-step together: bounds register pressure
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The loop body is one straight-line block: the loads of the next group are
  // issued before the current group's MFMAs and cannot be sunk next to their
  // use. A group past the end (odd count) loads clamped addresses and is
  // fully masked.
  xload(0);
  wload(0, WA);
  xstore(buf0);
  lds_barrier();
  for (int g = 0; g < ngroups; g += 2) {
    xload(g + 1);
    wload(g + 1, WB);
    compute(g, WA, buf0);
    xstore(buf1);
    lds_barrier();
    xload(g + 2);
    wload(g + 2, WA);
    compute(g + 1, WB, buf1);
    xstore(buf0);
    lds_barrier();
  }
}

template <int WT, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* buf0 = lds;
  char* buf1 = lds + kBufBytes;
  __shared__ int xrow_l[64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // block -> (split, column tile, row block, group); one 64-row block per
  // workgroup, so the workgroups of a tile stream its W concurrently
  int bid = blockIdx.x;
  const int s = bid % a.S;
  bid /= a.S;
  const int nb = bid % a.n_tiles;
  bid /= a.n_tiles;
  const int rb = bid % a.rb_stride;
  const int grp = bid / a.rb_stride;

  int r0 = 0, nrows = a.n_rows;
  if (a.group_off) {
    r0 = a.group_off[grp];
    nrows = a.group_off[grp + 1] - r0;
  }
  if (nrows <= rb * 64) return;

  constexpr int KS = WTraits<WT>::ks;
  const int nks_total = a.K / KS;
  const int ks0 = (int)((long long)s * nks_total / a.S);
  const int ks1 = (int)((long long)(s + 1) * nks_total / a.S);
  const int nks = ks1 - ks0;

  const int c_lane = wave * 16 + (lane & 15);
  const int wrow = w_row_of<EPI>(a, nb, c_lane);
  const bool wvalid = wrow < w_rows_total<EPI>(a);
  const char* wp = (const char*)a.W +
                   ((long long)grp * a.w_gstride + (long long)(wvalid ? wrow : 0) * a.K) * WTraits<WT>::esz +
                   (long long)ks0 * kStepBytes + (lane >> 4) * 16;   // this split's first k-step

  {
    const int rows_here = min(64, nrows - rb * 64);
    const int mtiles = (rows_here + 15) >> 4;
    if (tid < 64) {
      const int orow = r0 + rb * 64 + min(tid, rows_here - 1);   // clamp padding rows to a real row
      xrow_l[tid] = a.row_src ? a.row_src[orow] : orow;
    }
    __syncthreads();
    const char* xsrc = (const char*)a.X + (long long)xrow_l[tid >> 2] * a.x_ld * WTraits<WT>::esz;

    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nks > 0) {
      if (mtiles == 1) mainloop<WT, 1>(a, wp, wvalid, ks0, nks, xsrc, buf0, buf1, acc);
      else if (mtiles == 2) mainloop<WT, 2>(a, wp, wvalid, ks0, nks, xsrc, buf0, buf1, acc);
      else mainloop<WT, 4>(a, wp, wvalid, ks0, nks, xsrc, buf0, buf1, acc);
    }

    if constexpr (EPI == EPI_PARTIAL) {
      // row-major fp32 partial tile [64][64] of split s
      const long long tile_id = ((long long)grp * a.n_tiles + nb) * a.rb_stride + rb;
      float* pt = a.part + (tile_id * a.S + s) * 4096;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int m = mt * 16 + (lane & 15);
        if (m < rows_here)
          *reinterpret_cast<f32x4*>(pt + m * 64 + wave * 16 + (lane >> 4) * 4) = acc[mt];
      }
    } else {
      // finished tile -> LDS (reuses the X buffers: the last barrier ended all reads)
      float* T = (float*)lds;
      float wsc[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (WT == DT_E4M3) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int wr = w_row_of<EPI>(a, nb, wave * 16 + (lane >> 4) * 4 + r);
          wsc[r] = wr < w_rows_total<EPI>(a) ? a.w_scale[(long long)grp * a.ws_gstride + wr] : 0.f;
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int m = mt * 16 + (lane & 15);
        float xs = 1.f;
        if constexpr (WT == DT_E4M3) xs = a.x_scale[xrow_l[m]];
#pragma unroll
        for (int r = 0; r < 4; ++r) T[m * kTilePitch + wave * 16 + (lane >> 4) * 4 + r] = acc[mt][r] * wsc[r] * xs;
      }
      __syncthreads();
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
      } else if constexpr (EPI == EPI_SWIGLU) {
        if (rvalid && cq < 32) {
          const int j0 = nb * 32 + cq;
          float z[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float g = trow[cq + i], u = trow[32 + cq + i];
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
            for (int i = 0; i < 16; i += 4) *reinterpret_cast<f32x4*>(o + i) = f32x4{z[i], z[i + 1], z[i + 2], z[i + 3]};
          }
        }
      }
    }
  }
}

template <int WT, int EPI>
static hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  const int grid = a.n_tiles * a.n_groups * a.rb_stride * a.S;
  hipLaunchKernelGGL((k_gemm<WT, EPI>), dim3(grid), dim3(256), kGemmLds, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int wt, int epi, const GemmArgs& a, hipStream_t st) {
#define SPA_CASE(W, E) \
  if (wt == W && epi == E) return launch_t<W, E>(a, st);
  SPA_CASE(DT_BF16, EPI_PARTIAL)
  SPA_CASE(DT_F32, EPI_PARTIAL)
  SPA_CASE(DT_E4M3, EPI_PARTIAL)
  SPA_CASE(DT_BF16, EPI_SWIGLU)
  SPA_CASE(DT_F32, EPI_SWIGLU)
  SPA_CASE(DT_E4M3, EPI_SWIGLU)
  SPA_CASE(DT_BF16, EPI_STORE)
  SPA_CASE(DT_F32, EPI_STORE)
  SPA_CASE(DT_E4M3, EPI_STORE)
#undef SPA_CASE
  return hipErrorInvalidValue;
}

int gemm_lds_bytes() { return kGemmLds; }

}  // namespace spa
