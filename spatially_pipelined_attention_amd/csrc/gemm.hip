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
#include "gemm_tile.h"

namespace spa {

// resident workgroups per CU the register budget is sized for
#ifndef SPA_GEMM_MINB
#define SPA_GEMM_MINB 2
#endif

template <int WT, int EPI, int CT, int MT>
__global__ __launch_bounds__(256, SPA_GEMM_MINB) void k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char red[gemm_red_bytes<CT, MT>()];
  gemm_tile<WT, EPI, CT, MT>(a, blockIdx.x, threadIdx.x, red);
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
