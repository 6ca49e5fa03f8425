// The weight-streaming GEMM tile (the body of k_gemm in gemm.hip) as a device
// function over an explicit block id, so a persistent kernel can run the same
// tiles with the same arithmetic: 256 threads (tid 0..255, 4 waves), LDS
// reduction buffer `red` of gemm_red_bytes<CT, MT>() bytes. Every thread of the
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

// The tile's finish: small tiles put all their row tiles in LDS at once
// (4 waves x MT x CT fragments of 1 KB, at most 32 KB), larger ones one row
// tile at a time through two alternating buffers.
template <int CT, int MT>
constexpr bool gemm_finish_at_once() { return 4 * MT * CT * 1024 <= 32 * 1024; }
template <int CT, int MT>
constexpr int gemm_red_bytes() { return gemm_finish_at_once<CT, MT>() ? 4 * MT * CT * 1024 : 2 * 4 * CT * 1024; }
// barriers one gemm_tile<.., CT, MT> call takes (a workgroup whose groups
// share barriers matches them when it has no tile)
template <int CT, int MT>
constexpr int gemm_tile_barriers() { return gemm_finish_at_once<CT, MT>() ? 2 : MT + 1; }

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
  float xsc[MT];   // E4M3: the activation scale of this lane's row of each row tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int orow = r0 + rb * BR + min(mt * 16 + lo16, rows_here - 1);   // padding rows repeat a real row
    const int src = a.row_src ? a.row_src[orow] : orow;
    xp[mt] = (const char*)a.X + (long long)src * a.x_rstride + (long long)ks0 * a.x_kstride + kq;
    xsc[mt] = 1.f;
    if constexpr (WT == DT_E4M3) xsc[mt] = a.x_scale[src];
  }

  // E4M3 weight channel scales of the fragments this wave will finish, also
  // loaded before the k-loop: slot u holds fragment f = wave + 4u (finished
  // a row tile at a time), or the fragment of pair wave + 4u (all row tiles
  // at once); its columns c4 + i (h = 1: the SwiGLU up partner)
  constexpr int NF = EPI == EPI_SWIGLU ? CT / 2 : CT;   // fragments (SwiGLU: gate/up pairs) to finish
  constexpr int NU = (NF + 3) / 4;                      // per wave, a row tile at a time
  constexpr int NS = gemm_finish_at_once<CT, MT>() ? (MT * NF + 3) / 4 : NU;
  const int c4 = (lane >> 4) * 4;                       // a lane holds row lo16, columns c4 .. c4 + 3 of a fragment
  float wsc[NS][2][4];
#pragma unroll
  for (int u = 0; u < NS; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) wsc[u][h][i] = 1.f;
  if constexpr (WT == DT_E4M3) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int pair = wave + 4 * u;
      int f = pair;
      if constexpr (gemm_finish_at_once<CT, MT>()) {
        if (pair >= MT * NF) continue;
        f = pair % NF;
      } else if (f >= NF) {
        continue;
      }
#pragma unroll
      for (int h = 0; h < (EPI == EPI_SWIGLU ? 2 : 1); ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int wr = w_row_of<EPI, CT>(a, nb, (f + h * (CT / 2)) * 16 + c4 + i);
          wsc[u][h][i] = wr < w_rows_total<EPI>(a) ? a.w_scale[(long long)grp * a.ws_gstride + wr] : 0.f;
        }
    }
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

  // Finish the tile: every wave puts its partial tiles in LDS, and the
  // (row tile, fragment) pairs are dealt over the 4 waves, each summed in
  // wave order (((w0 + w1) + w2) + w3) and finished (SwiGLU: gate fragment f
  // with its up partner f + CT/2). Small tiles go through LDS at once; larger
  // ones 16 rows at a time, wave w taking fragments w, w + 4, ..., through
  // two alternating buffers, so one barrier per row tile suffices: a buffer
  // is written again two row tiles later, after a barrier every wave reaches
  // only once its reads are done.
  // at once: [4 waves][MT][CT][64 lanes]; by row tile: [2][4 waves][CT][64 lanes]
  f32x4* rd = reinterpret_cast<f32x4*>(red);
  // finish fragment f (a gate/up pair for SwiGLU) of row tile mt from the 4
  // waves' copies at buf[(w * wstride + ct) * 64 + lane], with the scales of
  // slot u and the activation scale xs
  auto finish = [&](const f32x4* buf, int wstride, int mt, int f, int u, float xs) {
    const int m = mt * 16 + lo16;
    if (m >= rows_here) return;   // padding rows are not written
    const long long orow = r0 + rb * BR + m;
    f32x4 v[2];
#pragma unroll
    for (int h = 0; h < (EPI == EPI_SWIGLU ? 2 : 1); ++h) {
      const int ct = f + h * (CT / 2);
      f32x4 t = buf[ct * 64 + lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) t += buf[(w * wstride + ct) * 64 + lane];
      v[h] = t;
    }
    const float (&sc)[2][4] = wsc[u];
    if constexpr (EPI == EPI_PARTIAL) {
      // split s, row (dispatch or token row), padded column: [S][part_rows][part_ld];
      // every split is scaled, so the splits' sum is the scaled product
      f32x4 t = v[0];
      if constexpr (WT == DT_E4M3) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] *= sc[0][i] * xs;
      }
      float* pt = a.part + ((long long)s * a.part_rows + orow) * a.part_ld + nb * TC + f * 16 + c4;
      *reinterpret_cast<f32x4*>(pt) = t;
    } else if constexpr (EPI == EPI_STORE) {
      float o4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = v[0][i] * sc[0][i] * xs;
      float* o = (float*)a.out + orow * a.out_ld;
      const int c = nb * TC + f * 16 + c4;
      if (c + 3 < a.N) {
        *reinterpret_cast<f32x4*>(o + c) = f32x4{o4[0], o4[1], o4[2], o4[3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c + i < a.N) o[c + i] = o4[i];
      }
    } else {   // SwiGLU: fragment f < CT/2 holds gate columns, f + CT/2 the matching up columns
      const int j0 = nb * 8 * CT + f * 16 + c4;
      if (j0 >= a.inter) return;
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = v[0][i] * sc[0][i] * xs, up = v[1][i] * sc[1][i] * xs;
        z[i] = g / (1.0f + __expf(-g)) * up;
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
  };
  if constexpr (gemm_finish_at_once<CT, MT>()) {
    // [4 waves][MT][CT][64 lanes]; pair i = (mt, f) goes to wave i % 4
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) rd[((wave * MT + mt) * CT + ct) * 64 + lane] = acc[mt][ct];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (MT * NF + 3) / 4; ++i) {
      const int pair = wave + 4 * i;
      if (pair < MT * NF) {
        const int mt = pair / NF, f = pair - mt * NF;
        float xs = xsc[0];   // xsc[mt] without a dynamic register index
#pragma unroll
        for (int j = 1; j < MT; ++j) xs = mt == j ? xsc[j] : xs;
        finish(rd + mt * CT * 64, MT * CT, mt, f, i, xs);   // wave w's copy of row tile mt: MT * CT fragments apart
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4* buf = rd + (mt & 1) * 4 * CT * 64;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) buf[(wave * CT + ct) * 64 + lane] = acc[mt][ct];
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int f = wave + 4 * u;
        if (f < NF) finish(buf, CT, mt, f, u, xsc[mt]);
      }
    }
  }
  __syncthreads();   // the LDS buffers are free again when the call returns
}

}  // namespace spa
