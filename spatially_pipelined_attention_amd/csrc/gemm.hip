// Skinny matrix products of the decode layer on gfx950 MFMA.
//
// Every projection of the layer (Figure 3 of the SubGPU Pipelining paper:
// Q/KV projection, output projection, router gating, expert up, expert down)
// is Y[r][n] = sum_k X[r][k] * W[n][k] with few rows r (the decoded tokens of
// a microbatch, or the rows routed to one expert) and a large W read once
// from HBM. The kernel is a weight stream:
//   * a workgroup owns 64 output columns of one block of up to 16*MT rows
//     (one W read serves all rows of the block); its 4 waves take the
//     k-steps of the workgroup's K range round-robin (wave w: steps w, w+4,
//     ...), so together they walk each W row front to back;
//   * each wave keeps a ring of P k-steps of W and X fragments in flight in
//     registers (W straight from HBM, X from L2) and multiplies the oldest;
//     the hot loop has no barriers and no data-dependent branches (steps past
//     the end load a clamped address and are masked to zero);
//   * at the end the 4 wave tiles are summed in wave order through LDS, one
//     16-row tile at a time, and wave 0 writes the result: an fp32 partial
//     tile for a split-K finish kernel (the k range may be split over S
//     workgroups, summed later in split order), or the finished rows, with
//     E4M3 per-row and per-channel scales applied, either stored plainly or
//     through SwiGLU (a tile's columns 0-31 are gate rows and 32-63 the
//     matching up rows, so gate and up of one output sit in the same lane).
// MFMA operand layout: A = W fragment (16 output columns x k), B = X
// fragment (k x 16 rows); lane l holds C[4(l/16)+i][l%16], i.e. output
// column 4(l/16)+i of the fragment for row l%16. Both operands take the k
// elements of a 64-byte k-step in the same lane order, so the product is the
// plain dot product.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace spa {

constexpr int kStepBytes = 64;     // one k-step of one row
#ifndef SPA_GEMM_W_NT
#define SPA_GEMM_W_NT 1
#endif
constexpr bool kWStream = SPA_GEMM_W_NT != 0;   // weights are read once per launch: non-temporal loads

// ring depth: keeps the register budget of two workgroups per CU
#ifndef SPA_GEMM_RING_BIG
#define SPA_GEMM_RING_BIG 2
#endif
#ifndef SPA_GEMM_RING_MID
#define SPA_GEMM_RING_MID 3
#endif
template <int CT, int MT> struct Ring {
  static constexpr int P = CT * MT > 16 ? SPA_GEMM_RING_BIG : (CT * MT > 8 ? SPA_GEMM_RING_MID : 4);
};

// resident workgroups per CU the register budget is sized for
#ifndef SPA_GEMM_MINB
#define SPA_GEMM_MINB 2
#endif

template <int WT, int EPI, int CT, int MT>
__global__ __launch_bounds__(256, SPA_GEMM_MINB) void k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char red[3 * CT * 64 * 16];   // wave reduction of one 16-row tile
  constexpr int P = Ring<CT, MT>::P;
  constexpr int BR = 16 * MT;
  constexpr int TC = 16 * CT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int s, nb, grp, rb, r0, nrows;
  if (!gemm_block(a, BR, lane, &s, &nb, &grp, &rb, &r0, &nrows)) return;
  const int blk = rb;   // rotation seed
  const int rows_here = min(BR, nrows - rb * BR);

  constexpr int KS = WTraits<WT>::ks;
  constexpr int esz = WTraits<WT>::esz;
  const int nks_total = a.K / KS;
  const int ks0 = (int)((long long)s * nks_total / a.S);
  const int nks = (int)((long long)(s + 1) * nks_total / a.S) - ks0;

  // per-lane fragment base pointers. W is stored in 16-row panels: panel p
  // holds rows 16p..16p+15 as [k-step][16 rows][64 bytes], so the fragment of
  // one k-step is 1 KB of contiguous memory
  const int lo16 = lane & 15, kq = (lane >> 4) * 16;
  const long long panel_bytes = (long long)nks_total * 1024;
  const char* wp[CT];
  bool wvalid[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int wrow0 = w_row_of<EPI, CT>(a, nb, ct * 16);            // first row of the fragment (16-aligned)
    wvalid[ct] = wrow0 + lo16 < w_rows_total<EPI>(a);
    wp[ct] = (const char*)a.W + (long long)grp * a.w_gstride * esz + (long long)((wvalid[ct] ? wrow0 : 0) >> 4) * panel_bytes +
             (long long)ks0 * 1024 + lo16 * 64 + kq;
  }
  // X fragment of row-tile mt: 16 rows of one k-step; rows sit x_rstride
  // bytes apart and k-steps x_kstride bytes apart (row-major or k-step-major)
  const char* xp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int orow = r0 + rb * BR + min(mt * 16 + lo16, rows_here - 1);   // padding rows repeat a real row
    const int src = a.row_src ? a.row_src[orow] : orow;
    xp[mt] = (const char*)a.X + (long long)src * a.x_rstride + (long long)ks0 * a.x_kstride + kq;
  }

  f32x4 acc[MT][CT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nks > 0) {
    u32x4 Wr[P][CT], Xr[P][MT];
    const u32x4 zero = {0u, 0u, 0u, 0u};
#ifndef SPA_GEMM_ALL_TILES
#define SPA_GEMM_ALL_TILES 0
#endif
    const int mt_live = SPA_GEMM_ALL_TILES ? MT : __builtin_amdgcn_readfirstlane((rows_here + 15) >> 4);
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) Xr[p][mt] = zero;
    // Wave w takes k-steps w + 4g of this split; the workgroups of a product
    // start at different groups g (a rotation fixed by the tile), so they do
    // not all read the same X lines at once. Summation order stays fixed.
    const int kl = nks - 1;
    const int ng = (nks + 3) / 4;                  // groups of 4 k-steps
    const int rot = (int)(((unsigned)nb * 7u + (unsigned)blk * 13u) % (unsigned)ng);
    auto kstep = [&](int j) {
      int g = j + rot;
      g = g >= ng ? g - ng : g;
      return j < ng ? min(wave + 4 * g, kl) : kl;
    };
    auto load = [&](int slot, int j) {
      const long long kk = kstep(j);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) Wr[slot][ct] = kWStream ? ld16_stream(wp[ct] + kk * 1024) : ld16(wp[ct] + kk * 1024);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < mt_live) Xr[slot][mt] = ld16(xp[mt] + kk * a.x_kstride);
    };
    auto compute = [&](int slot, int j) {
      int g = j + rot;
      g = g >= ng ? g - ng : g;
      const bool live = j < ng && wave + 4 * g < nks;   // wave-uniform
      u32x4 w[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) w[ct] = (live && wvalid[ct]) ? Wr[slot][ct] : zero;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < mt_live) {   // row tiles past the block's rows hold only padding
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) acc[mt][ct] = mma_step<WT>(w[ct], Xr[slot][mt], acc[mt][ct]);
        }
    };
    // groups rounded up to the ring depth
    const int J = (ng + P - 1) / P * P;
#pragma unroll
    for (int p = 0; p < P; ++p) load(p, p);
    // straight-line rounds: multiply slot p, then refill it P steps ahead; the
    // scheduling barriers keep each refill right behind its multiply so the
    // wave always has P-1 k-steps of loads in flight
    for (int j0 = 0; j0 + P < J; j0 += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        compute(p, j0 + p);
        __builtin_amdgcn_sched_barrier(0);
        load(p, j0 + P + p);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) compute(p, J - P + p);
  }

  // sum the wave tiles in wave order: 16 rows at a time through LDS
  f32x4* rd = reinterpret_cast<f32x4*>(red);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (wave > 0) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) rd[((wave - 1) * CT + ct) * 64 + lane] = acc[mt][ct];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[mt][ct] += rd[(w * CT + ct) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;

  // wave 0 holds the tile: row mt*16 + lo16, columns ct*16 + c4 + i
  const int c4 = (lane >> 4) * 4;
  // E4M3: per-output-channel weight scales and per-row activation scales
  float wsc[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) wsc[ct][i] = 1.f;
  if constexpr (WT == DT_E4M3) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int wr = w_row_of<EPI, CT>(a, nb, ct * 16 + c4 + i);
        wsc[ct][i] = wr < w_rows_total<EPI>(a) ? a.w_scale[(long long)grp * a.ws_gstride + wr] : 0.f;
      }
  }
  if constexpr (EPI == EPI_PARTIAL) {
    // split s, row (dispatch or token row), padded column: [S][part_rows][part_ld];
    // every split is scaled, so the splits' sum is the scaled product
    float* pt = a.part + ((long long)s * a.part_rows + r0 + rb * BR) * a.part_ld + nb * TC + c4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + lo16;
      if (m < rows_here) {
        float xs = 1.f;
        if constexpr (WT == DT_E4M3) {
          const long long orow = r0 + rb * BR + m;
          xs = a.x_scale[a.row_src ? a.row_src[orow] : orow];
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          f32x4 v = acc[mt][ct];
          if constexpr (WT == DT_E4M3) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] *= wsc[ct][i] * xs;
          }
          *reinterpret_cast<f32x4*>(pt + (long long)m * a.part_ld + ct * 16) = v;
        }
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + lo16;
      if (m >= rows_here) continue;
      const long long orow = r0 + rb * BR + m;
      float xs = 1.f;
      if constexpr (WT == DT_E4M3) xs = a.x_scale[a.row_src ? a.row_src[orow] : orow];
      float v[CT][4];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[ct][i] = acc[mt][ct][i] * wsc[ct][i] * xs;
      if constexpr (EPI == EPI_STORE) {
        float* o = (float*)a.out + orow * a.out_ld;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int c = nb * TC + ct * 16 + c4;
          if (c + 3 < a.N) {
            *reinterpret_cast<f32x4*>(o + c) = f32x4{v[ct][0], v[ct][1], v[ct][2], v[ct][3]};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (c + i < a.N) o[c + i] = v[ct][i];
          }
        }
      } else {   // SwiGLU: fragments ct < CT/2 are gate columns, ct + CT/2 the matching up columns
#pragma unroll
        for (int ct = 0; ct < CT / 2; ++ct) {
          const int j0 = nb * 8 * CT + ct * 16 + c4;
          if (j0 >= a.inter) continue;
          float z[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float g = v[ct][i], u = v[ct + CT / 2][i];
            z[i] = g / (1.0f + __expf(-g)) * u;
          }
          const long long zr = a.out_kmajor_rows;
          if (a.out_dtype == DT_BF16) {   // k-step-major: 32 bf16 per k-step
            uint16_t* o = (uint16_t*)a.out + (zr ? ((long long)(j0 >> 5) * zr + orow) * 32 + (j0 & 31) : orow * a.out_ld + j0);
            *reinterpret_cast<uint2*>(o) = uint2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
          } else {                        // k-step-major: 16 fp32 per k-step
            float* o = (float*)a.out + (zr ? ((long long)(j0 >> 4) * zr + orow) * 16 + (j0 & 15) : orow * a.out_ld + j0);
            *reinterpret_cast<f32x4*>(o) = f32x4{z[0], z[1], z[2], z[3]};
          }
        }
      }
    }
  }
}

template <int WT, int EPI, int CT, int MT>
static hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  const int grid = a.n_tiles * a.rb_stride * a.S;
  hipLaunchKernelGGL((k_gemm<WT, EPI, CT, MT>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int WT, int EPI, int CT>
static hipError_t launch_mt(const GemmArgs& a, hipStream_t st) {
  switch (a.blk_rows) {
    case 16: return launch_t<WT, EPI, CT, 1>(a, st);
    case 32: return launch_t<WT, EPI, CT, 2>(a, st);
    case 48: return launch_t<WT, EPI, CT, 3>(a, st);
    case 64: return launch_t<WT, EPI, CT, 4>(a, st);
    case 80: return launch_t<WT, EPI, CT, 5>(a, st);
    case 128: return launch_t<WT, EPI, CT, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int WT, int EPI>
static hipError_t launch_ct(const GemmArgs& a, hipStream_t st) {
  if (a.tile_cols == 64) return launch_mt<WT, EPI, 4>(a, st);
  if constexpr (WT != DT_F32) {
    if (a.tile_cols == 32) return launch_mt<WT, EPI, 2>(a, st);
    if (a.tile_cols == 96) return launch_mt<WT, EPI, 6>(a, st);
    if constexpr (EPI != EPI_SWIGLU)   // SwiGLU tiles pair gate and up halves: an even fragment count
      if (a.tile_cols == 48) return launch_mt<WT, EPI, 3>(a, st);
  } else if constexpr (EPI == EPI_PARTIAL) {
    if (a.tile_cols == 16) return launch_mt<WT, EPI, 1>(a, st);   // the router: few outputs, many workgroups
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int wt, int epi, const GemmArgs& a, hipStream_t st) {
  if (a.group_off && a.n_groups > 128) return hipErrorInvalidValue;   // the block scan holds 2 groups per lane
  if (a.tile_cols == 128) return launch_gemm_big(wt, epi, a, st);    // 128-row blocks: the LDS-tiled kernel
#define SPA_CASE(W, E) \
  if (wt == W && epi == E) return launch_ct<W, E>(a, st);
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

bool gemm_blk_rows_ok(int r) { return r == 16 || r == 32 || r == 48 || r == 64 || r == 80 || r == 128; }

}  // namespace spa
