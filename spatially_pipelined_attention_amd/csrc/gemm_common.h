// Helpers of the skinny-GEMM kernel (gemm.hip): MFMA steps per weight type,
// the weight row of a tile column, and the workgroup -> tile mapping.
#pragma once
#include "common.h"
#include "kernels.h"

namespace spa {

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

// W row feeding tile column c (0..16*CT-1) of column tile nb; a SwiGLU tile
// pairs 8*CT gate rows with the 8*CT up rows of the same outputs.
template <int EPI, int CT>
__device__ __forceinline__ int w_row_of(const GemmArgs& a, int nb, int c) {
  constexpr int HC = 8 * CT;
  if constexpr (EPI == EPI_SWIGLU) return c < HC ? nb * HC + c : a.inter + nb * HC + (c - HC);
  else return nb * 16 * CT + c;
}

template <int EPI>
__device__ __forceinline__ int w_rows_total(const GemmArgs& a) {
  if constexpr (EPI == EPI_SWIGLU) return 2 * a.inter;
  else return a.N;
}

// Workgroup -> (split s, column tile nb, group grp, row block rb, first row
// r0 of the group, rows of the group). Grouped products number the non-empty
// row blocks of all groups in group order (wave-parallel scan of the per-group
// block counts, two groups per lane). Returns false when the workgroup has no
// rows (the whole workgroup returns: the result is wave-uniform).
__device__ __forceinline__ bool gemm_block(const GemmArgs& a, int BR, int lane, int bid, int* s_out, int* nb_out,
                                           int* grp_out, int* rb_out, int* r0_out, int* nrows_out) {
  const int s = bid % a.S;
  bid /= a.S;
  const int nb = bid % a.n_tiles;
  const int blk = bid / a.n_tiles;
  int grp = 0, rb = blk, r0 = 0, nrows = a.n_rows;
  if (a.group_off) {
    const int g0 = 2 * lane, g1 = 2 * lane + 1;
    // offsets of this lane's two groups and of the one after them (kept: the
    // chosen group's first row comes from its lane, not from another load)
    const int o0 = g0 <= a.n_groups ? a.group_off[g0] : 0;
    const int o1 = g1 <= a.n_groups ? a.group_off[g1] : 0;
    const int o2 = g1 + 1 <= a.n_groups ? a.group_off[g1 + 1] : 0;
    const int n0 = g0 < a.n_groups ? o1 - o0 : 0;
    const int n1 = g1 < a.n_groups ? o2 - o1 : 0;
    const int c0 = (n0 + BR - 1) / BR, c1 = (n1 + BR - 1) / BR;
    int incl = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const int excl = incl - c0 - c1;
    const unsigned long long hit = __ballot(blk >= excl && blk < incl);
    if (hit == 0ull) return false;                 // past the last non-empty block
    const int hl = __builtin_ctzll(hit);
    const int e = __shfl(excl, hl, 64), cc0 = __shfl(c0, hl, 64);
    const bool first = blk - e < cc0;   // the lane's first group
    grp = first ? 2 * hl : 2 * hl + 1;
    rb = first ? blk - e : blk - e - cc0;
    r0 = first ? __shfl(o0, hl, 64) : __shfl(o1, hl, 64);
    nrows = first ? __shfl(n0, hl, 64) : __shfl(n1, hl, 64);
    grp = __builtin_amdgcn_readfirstlane(grp);
    rb = __builtin_amdgcn_readfirstlane(rb);
    r0 = __builtin_amdgcn_readfirstlane(r0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
  }
  if (nrows <= rb * BR) return false;
  *s_out = s;
  *nb_out = nb;
  *grp_out = grp;
  *rb_out = rb;
  *r0_out = r0;
  *nrows_out = nrows;
  return true;
}

}  // namespace spa
