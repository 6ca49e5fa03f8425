// Projections with many rows per weight block on gfx950 MFMA (the expert and
// dense products of Figure 3 of the SubGPU Pipelining paper at large decode
// batches: hundreds of rows per expert).
//
// The weight-streaming kernel (gemm.hip) keeps both operands in registers and
// loads every fragment from memory once per workgroup; with 128 rows per
// block its activation loads outnumber the weight loads, and the per-CU load
// path, not the matrix cores, sets the pace. Here a workgroup owns a 128-row
// x 128-column tile and streams K through LDS:
//   * per 64-byte k-step the 256 threads load the block's 128 activation rows
//     and 128 weight rows (16 KB, four 16-byte loads per thread) into one of
//     two LDS buffers (one barrier per k-step); the loads are issued two
//     k-steps ahead into two register slots, so each has two k-steps of
//     multiplication to land before it is stored to LDS;
//   * the 4 waves form a 2 x 2 grid of 64 x 64 sub-tiles; each reads its 4
//     activation and 4 weight fragments from LDS and issues 16 MFMA tiles, so
//     every loaded byte feeds 64 output rows or columns instead of one tile;
//   * each output is summed in k order by one lane, over the workgroup's k
//     range (the whole of K, or split s of S for fp32 partials summed later
//     in split order); the epilogues are those of gemm.hip: fp32 rows (a
//     split partial, or the plain product) or SwiGLU, with E4M3 row and
//     channel scales. A SwiGLU tile holds 64 outputs: for each wave column
//     half, 32 gate rows followed by their 32 up rows, so gate and up of one
//     output meet in one lane.
// Operand layout as in gemm.hip: A = weight fragment (16 output columns x k),
// B = activation fragment (k x 16 rows); lane l holds C[4(l/16)+i][l%16].
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

#include <type_traits>

namespace spa {

constexpr int kBigRows = 128;     // activation rows per workgroup
constexpr int kBigCols = 128;     // weight rows per workgroup
constexpr int kLdsRow = 80;       // bytes per LDS row: a 64-byte k-step + 16 bytes against bank conflicts

template <int EPI>
__device__ __forceinline__ int big_wrow(const GemmArgs& a, int nb, int c) {
  if constexpr (EPI == EPI_SWIGLU) {
    const int half = c >> 6, j = c & 63;
    const int out = nb * 64 + half * 32 + (j & 31);
    return j < 32 ? out : a.inter + out;
  } else {
    return nb * kBigCols + c;
  }
}

template <int WT, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_big(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char xs[2][kBigRows * kLdsRow];
  __shared__ __attribute__((aligned(16))) char wsm[2][kBigCols * kLdsRow];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  int s, nb, grp, rb, r0, nrows;
  if (!gemm_block(a, kBigRows, lane, blockIdx.x, &s, &nb, &grp, &rb, &r0, &nrows)) return;
  const int rows_here = min(kBigRows, nrows - rb * kBigRows);

  constexpr int KS = WTraits<WT>::ks;
  constexpr int esz = WTraits<WT>::esz;
  const int nks_total = a.K / KS;
  const long long panel_bytes = (long long)nks_total * 1024;
  // split s of S (partials only): k-steps [ks0, ks0 + nks)
  const int ks0 = (int)((long long)s * nks_total / a.S);
  const int nks = (int)((long long)(s + 1) * nks_total / a.S) - ks0;
  const int wtotal = EPI == EPI_SWIGLU ? 2 * a.inter : a.N;

  // this thread's two activation and two weight chunks of a k-step: chunk q
  // (0..511) is 16 bytes `q & 3` of row / weight row `q >> 2`
  const char* xsrc[2];
  const char* wsrc[2];
  int ldsoff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = tid + 256 * h, row = q >> 2, part = q & 3;
    const int orow = r0 + rb * kBigRows + min(row, rows_here - 1);   // padding rows repeat a real row
    const int src = a.row_src ? a.row_src[orow] : orow;
    xsrc[h] = (const char*)a.X + (long long)src * a.x_rstride + (long long)ks0 * a.x_kstride + part * 16;
    const int wrow = big_wrow<EPI>(a, nb, row);
    const int wv = wrow < wtotal ? wrow : 0;   // rows past the matrix load row 0; their outputs are dropped
    wsrc[h] = (const char*)a.W + (long long)grp * a.w_gstride * esz + (long long)(wv >> 4) * panel_bytes +
              (long long)ks0 * 1024 + (wv & 15) * 64 + part * 16;
    ldsoff[h] = row * kLdsRow + part * 16;
  }
  // two register slots of one k-step each: the loads of k-step k + 2 go out
  // while k is multiplied, so every load has two k-steps of MFMA work to land
  u32x4 xr[2][2], wreg[2][2];
  auto load = [&](auto slot_c, int kk) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      xr[sl][h] = ld16(xsrc[h] + (long long)kk * a.x_kstride);
      wreg[sl][h] = ld16(wsrc[h] + (long long)kk * 1024);
    }
  };
  auto stash = [&](auto slot_c) {   // slot sl into LDS buffer sl
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<u32x4*>(&xs[sl][ldsoff[h]]) = xr[sl][h];
      *reinterpret_cast<u32x4*>(&wsm[sl][ldsoff[h]]) = wreg[sl][h];
    }
  };
  constexpr std::integral_constant<int, 0> S0{};
  constexpr std::integral_constant<int, 1> S1{};

  f32x4 acc[4][4];
#pragma unroll
  for (int mf = 0; mf < 4; ++mf)
#pragma unroll
    for (int cf = 0; cf < 4; ++cf) acc[mf][cf] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lo16 = lane & 15, kq = (lane >> 4) * 16;
  const int xrd = (wr * 64 + lo16) * kLdsRow + kq;   // fragment mf at + mf * 16 rows
  const int wrd = (wc * 64 + lo16) * kLdsRow + kq;

  // E4M3: this lane's weight channel scales and activation row scales, loaded
  // before the k-loop so that the epilogue does not wait for them
  // (lane: row wr*64 + mf*16 + lo16 of the block; tile column wc*64 + cf*16 + c4 + i)
  const int c4 = (lane >> 4) * 4;
  float wsc[4][4], xsc[4];
#pragma unroll
  for (int cf = 0; cf < 4; ++cf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wsc[cf][i] = 1.f;
      if constexpr (WT == DT_E4M3) {
        const int wrow = big_wrow<EPI>(a, nb, wc * 64 + cf * 16 + c4 + i);
        wsc[cf][i] = wrow < wtotal ? a.w_scale[(long long)grp * a.ws_gstride + wrow] : 0.f;
      }
    }
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
    xsc[mf] = 1.f;
    if constexpr (WT == DT_E4M3) {
      const long long orow = r0 + rb * kBigRows + min(wr * 64 + mf * 16 + lo16, rows_here - 1);
      xsc[mf] = a.x_scale[a.row_src ? a.row_src[orow] : orow];
    }
  }

  if (nks > 0) {
    load(S0, 0);
    stash(S0);
  }
  if (nks > 1) load(S1, 1);
  __syncthreads();
  // k-step k sits in LDS buffer and register slot k & 1
  auto step = [&](auto slot_c, int k) {
    constexpr int sl = decltype(slot_c)::value;
    if (k + 2 < nks) load(slot_c, k + 2);   // this slot's k-step was stashed one step ago
    u32x4 xf[4], wf[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      xf[f] = *reinterpret_cast<const u32x4*>(&xs[sl][xrd + f * 16 * kLdsRow]);
      wf[f] = *reinterpret_cast<const u32x4*>(&wsm[sl][wrd + f * 16 * kLdsRow]);
    }
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int cf = 0; cf < 4; ++cf) acc[mf][cf] = mma_step<WT>(wf[cf], xf[mf], acc[mf][cf]);
    if (k + 1 < nks) {   // k-step k + 1 into the other buffer (read one step ago by every wave)
      if constexpr (sl == 0) stash(S1);
      else stash(S0);
    }
    __syncthreads();
  };
  for (int k = 0; k < nks; k += 2) {
    step(S0, k);
    if (k + 1 < nks) step(S1, k + 1);
  }

#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
    const int m = wr * 64 + mf * 16 + lo16;
    if (m >= rows_here) continue;
    const long long orow = r0 + rb * kBigRows + m;
    const float xs = xsc[mf];
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int cf = 0; cf < 2; ++cf) {   // fragments 0, 1 gate; 2, 3 the matching up
        const int j0 = nb * 64 + wc * 32 + cf * 16 + c4;
        if (j0 >= a.inter) continue;
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[mf][cf][i] * wsc[cf][i] * xs, u = acc[mf][cf + 2][i] * wsc[cf + 2][i] * xs;
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
    } else {
      // split s of the partial buffer [S][part_rows][part_ld] (EPI_PARTIAL),
      // or the output rows (EPI_STORE, one split)
      float* o = EPI == EPI_PARTIAL ? a.part + ((long long)s * a.part_rows + orow) * a.part_ld
                                    : (float*)a.out + orow * a.out_ld;
      const int ncols = EPI == EPI_PARTIAL ? a.part_ld : a.N;
#pragma unroll
      for (int cf = 0; cf < 4; ++cf) {
        const int c = nb * kBigCols + wc * 64 + cf * 16 + c4;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[mf][cf][i] * wsc[cf][i] * xs;
        if (c + 3 < ncols) {
          *reinterpret_cast<f32x4*>(o + c) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c + i < ncols) o[c + i] = v[i];
        }
      }
    }
  }
}

template <int WT, int EPI>
static hipError_t launch_big_t(const GemmArgs& a, hipStream_t st) {
  const int grid = a.n_tiles * a.rb_stride * a.S;
  hipLaunchKernelGGL((k_gemm_big<WT, EPI>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_big(int wt, int epi, const GemmArgs& a, hipStream_t st) {
  if (a.S < 1 || (a.S > 1 && epi != EPI_PARTIAL) || a.blk_rows != kBigRows || a.tile_cols != kBigCols)
    return hipErrorInvalidValue;
  if (a.group_off && a.n_groups > 128) return hipErrorInvalidValue;
#define SPA_CASE(W, E) \
  if (wt == W && epi == E) return launch_big_t<W, E>(a, st);
  SPA_CASE(DT_BF16, EPI_PARTIAL)
  SPA_CASE(DT_E4M3, EPI_PARTIAL)
  SPA_CASE(DT_BF16, EPI_SWIGLU)
  SPA_CASE(DT_E4M3, EPI_SWIGLU)
  SPA_CASE(DT_BF16, EPI_STORE)
  SPA_CASE(DT_E4M3, EPI_STORE)
#undef SPA_CASE
  return hipErrorInvalidValue;
}

}  // namespace spa
