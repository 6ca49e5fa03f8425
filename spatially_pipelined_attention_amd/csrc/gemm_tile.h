// The weight-streaming GEMM tile (the body of k_gemm in gemm.hip) as a device
// function over an explicit block id, so a persistent kernel can run the same
// tiles with the same arithmetic: 256 threads (tid 0..255, 4 waves), LDS
// reduction buffer `red` of gemm_red_bytes<CT>() bytes. Every thread of the
// 256 calls it; the block's barriers are those of the calling workgroup.
#pragma once
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

template <int CT>
constexpr int gemm_red_bytes() { return 3 * CT * 64 * 16; }   // wave reduction of one 16-row tile

// P: k-steps per wave in the register ring (the order of the products does
// not depend on it; only the count of zero-weight padding steps at the end).
template <int WT, int EPI, int CT, int MT, int P = Ring<CT, MT>::P>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int bid, int tid, char* red) {
  constexpr int BR = 16 * MT;
  constexpr int TC = 16 * CT;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int s, nb, grp, rb, r0, nrows;
  if (!gemm_block(a, BR, lane, bid, &s, &nb, &grp, &rb, &r0, &nrows)) return;
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

}  // namespace spa
