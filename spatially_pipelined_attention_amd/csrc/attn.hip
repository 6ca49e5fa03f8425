// Grouped-query decode attention with sinks on gfx950 (the "FMHA" operator of
// Figure 3 of the SubGPU Pipelining paper; full and sliding-window layers as
// in its section 5.1).
//
// Work item = a piece of one (sequence, KV head) window: a range of its
// 32-position blocks. k_attn cuts a window of L positions into ceil(L / chunk)
// chunks of equal block counts; k_attn_dealt cuts the launch's blocks into
// equal ranges (see there). The 4 waves of a workgroup take the blocks of
// their piece round-robin:
//   * S^T[pos][head] = K Q^T on MFMA: the K block streams from HBM straight
//     into A-operand registers (16 B per lane per 16x32 tile half), all query
//     heads of the KV group ride in the 16 B-operand columns;
//   * online softmax in base 2, one head per lane column, running max shared
//     by the 4 lanes that hold the column;
//   * O^T[d][head] += V^T P^T on MFMA: V is cached d-major inside each
//     32-position block (positions interleaved by v_slot) so the A operand is
//     again one contiguous 16 B load, and the lane's own probabilities are
//     exactly its B operand;
//   * each wave keeps two blocks of K/V in registers and always consumes the
//     older one first, so the next block's loads stay in flight;
//   * the 4 wave states merge through LDS; when the piece is the whole
//     window the sink is applied and o written at once, otherwise the piece's
//     (m, l, o) partial goes to workspace and k_attn_merge combines the pieces
//     in window order together with the sink logit:
//     M = max(sink, m_c), Z = 2^(sink-M) + sum l_c 2^(m_c-M), o = sum o_c 2^(m_c-M) / Z.
// Cache layouts (element offsets, D = 64):
//   packed (full layers):  region(seq, g) = (kv_off[seq] * Hkv + g * cap[seq]) * D
//   ring (sliding layers): region(seq, g) = (seq * Hkv + g) * W * D, slot = pos % W
//   K at region + k_offset(slot, d, 64 / element size) (32-slot blocks of
//     64-byte column groups, slot-major inside a group)
//   V at region + (slot / 32) * 32 * D + d * 32 + v_slot(slot % 32)
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace spa {

constexpr int kD = 64;

struct KvLoc {
  long long base;
  int n_valid;
  bool ok;
};

__device__ __forceinline__ KvLoc kv_locate(const AttnArgs& a, int seq, int g, int kind) {
  KvLoc r;
  const int L = a.kv_len[seq];
  if (kind == KV_RING) {
    r.base = ((long long)seq * a.n_kv_heads + g) * a.window * kD;
    r.n_valid = min(L, a.window);
    r.ok = L >= 1;
  } else {
    const int cap = a.kv_cap[seq];
    r.base = (a.kv_off[seq] * a.n_kv_heads + (long long)g * cap) * kD;
    r.n_valid = L;
    r.ok = L >= 1 && L <= cap;
  }
  return r;
}

// Element offset of o[token b][head hq][d]: row-major [n_tok][Hq * D], or
// k-step-major over o_kmajor_rows rows (64-byte k-steps of 32 bf16 / 16 fp32)
__device__ __forceinline__ long long o_index(const AttnArgs& a, int b, int hq, int d) {
  const int c = hq * kD + d;
  if (a.o_kmajor_rows > 0) {
    const int ks = a.kv_dtype == DT_BF16 ? 32 : 16;
    return ((long long)(c / ks) * a.o_kmajor_rows + b) * ks + c % ks;
  }
  return (long long)b * a.n_q_heads * kD + c;
}

template <int KVT>
struct BlockRegs;

template <>
struct BlockRegs<DT_BF16> {
  u32x4 k[2][2];   // [tile][d half]
  u32x4 v[4];      // [d tile]
};

template <>
struct BlockRegs<DT_F32> {
  u32x4 k[2][4];   // [tile][d quarter]
  u32x4 v[4][2];   // [d tile][slot half]
};

template <int KVT>
__device__ __forceinline__ void load_block(BlockRegs<KVT>& br, const char* kreg, const char* vreg, int blk, int lane,
                                           bool stream) {
  const int p16 = lane & 15, q4 = lane >> 4;
  if constexpr (KVT == DT_BF16) {
    const char* kb = kreg + ((long long)blk * 32 * kD) * 2;
    const char* vb = vreg + ((long long)blk * 32 * kD) * 2;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const char* p = kb + (32 * 32 * h + (16 * t + p16) * 32 + 8 * q4) * 2;
        br.k[t][h] = stream ? ld16_stream(p) : ld16(p);
      }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const char* p = vb + ((16 * dt + p16) * 32 + 8 * q4) * 2;
      br.v[dt] = stream ? ld16_stream(p) : ld16(p);
    }
  } else {
    const char* kb = kreg + ((long long)blk * 32 * kD) * 4;
    const char* vb = vreg + ((long long)blk * 32 * kD) * 4;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const char* p = kb + (32 * 16 * cc + (16 * t + p16) * 16 + 4 * q4) * 4;
        br.k[t][cc] = stream ? ld16_stream(p) : ld16(p);
      }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* p = vb + ((16 * dt + p16) * 32 + 8 * q4 + 4 * hh) * 4;
        br.v[dt][hh] = stream ? ld16_stream(p) : ld16(p);
      }
  }
}

template <int KVT>
struct QRegs;
template <>
struct QRegs<DT_BF16> { u32x4 q[2]; };
template <>
struct QRegs<DT_F32> { u32x4 q[4]; };

// One 32-position block: scores, online softmax update, PV accumulation.
// MASK: the block holds positions at or past n_valid (the sequence's last
// block); only then are scores and V rows masked. exp2 is the hardware
// instruction: its arguments are <= 0 here, and -inf gives 0.
template <int KVT, bool MASK>
__device__ __forceinline__ void attend_block(const BlockRegs<KVT>& br, const QRegs<KVT>& qr, int blk, int n_valid,
                                             float scale_log2, float& m_run, float& l_run, f32x4 (&acc)[4],
                                             int lane) {
  const int q4 = lane >> 4;
  f32x4 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (KVT == DT_BF16) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(br.k[t][h]), bitcast<bf16x8>(qr.q[h]), s[t],
                                                      0, 0, 0);
    } else {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          s[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(br.k[t][cc][u]), __uint_as_float(qr.q[cc][u]),
                                                     s[t], 0, 0, 0);
    }
  }
  // scale (+ mask); this lane holds positions 16t + 4q4 + r of head (lane & 15)
  const int pos0 = blk * 32;
  float bmax = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = s[t][r] * scale_log2;
      if constexpr (MASK) v = pos0 + 16 * t + 4 * q4 + r < n_valid ? v : -INFINITY;
      s[t][r] = v;
      bmax = fmaxf(bmax, v);
    }
  bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
  bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
  const float m_new = fmaxf(m_run, bmax);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // m_run = -inf on the first block -> 0
  m_run = m_new;
  float p[2][4];
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[t][r] = __builtin_amdgcn_exp2f(s[t][r] - m_new);
      psum += p[t][r];
    }
  l_run = l_run * alpha + psum;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;

  if constexpr (KVT == DT_BF16) {
    u32x4 pf = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]), pack_bf16x2(p[1][0], p[1][1]),
                pack_bf16x2(p[1][2], p[1][3])};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      u32x4 vv = br.v[dt];
      if constexpr (MASK) {   // zero V of the masked positions (their cache rows may hold anything)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // word w holds slots 8q4 + 2w, 8q4 + 2w + 1
          int u0 = 2 * w, u1 = 2 * w + 1;
          int pa = pos0 + (u0 < 4 ? 4 * q4 + u0 : 16 + 4 * q4 + u0 - 4);
          int pb = pos0 + (u1 < 4 ? 4 * q4 + u1 : 16 + 4 * q4 + u1 - 4);
          uint32_t m = (pa < n_valid ? 0x0000ffffu : 0u) | (pb < n_valid ? 0xffff0000u : 0u);
          vv[w] &= m;
        }
      }
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(vv), bitcast<bf16x8>(pf), acc[dt], 0, 0, 0);
    }
  } else {
    float pv[8] = {p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float vv = __uint_as_float(br.v[dt][u >> 2][u & 3]);
        if constexpr (MASK) {
          int pp = pos0 + (u < 4 ? 4 * q4 + u : 16 + 4 * q4 + u - 4);
          vv = pp < n_valid ? vv : 0.f;
        }
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, pv[u], acc[dt], 0, 0, 0);
      }
  }
}

// The block's positions reach past n_valid only in the sequence's last block
// (a wave-uniform test): that one takes the masked variant.
template <int KVT>
__device__ __forceinline__ void attend(const BlockRegs<KVT>& br, const QRegs<KVT>& qr, int blk, int n_valid,
                                       float scale_log2, float& m_run, float& l_run, f32x4 (&acc)[4], int lane) {
  if (blk * 32 + 32 > n_valid)
    attend_block<KVT, true>(br, qr, blk, n_valid, scale_log2, m_run, l_run, acc, lane);
  else
    attend_block<KVT, false>(br, qr, blk, n_valid, scale_log2, m_run, l_run, acc, lane);
}

// minimum resident workgroups per CU (caps the registers per lane)
#ifndef SPA_ATTN_MINB
#define SPA_ATTN_MINB 2
#endif
#ifndef SPA_ATTN_RING
#define SPA_ATTN_RING 2
#endif
constexpr int kRing = SPA_ATTN_RING;   // 32-position blocks in registers per wave

// KIND (ring or packed cache) is a template parameter so that sliding and
// full layers are distinct kernels in profiles.
struct AttnLds {
  float m[4][16];
  float l[4][16];
  float o[4][kD][17];
};

#ifndef SPA_ATTN_NT
#define SPA_ATTN_NT 1
#endif
constexpr bool kStreamKV = SPA_ATTN_NT != 0;   // KV is read once: non-temporal loads

// ---------------------------------------------------------------------------
// The QKV finish folded into the attention (bf16 KV, 8 query heads per KV
// head, at most kFoldMaxSplits QKV splits). A wave that attends window
// (token b, KV group g) sums its group's q and the window's new K and V from
// the QKV split partials itself, with the finish kernel's arithmetic, and
// patches the new K/V into the registers of the block that holds the new slot
// (that block's load may return the slot's old row); the wave that attends
// that block also appends them to the cache. The values attended are the ones
// the finish kernel would have stored.

// The group's partials of one split, read contiguously, 16 bytes per lane: q
// of its 8 heads as two 1 KB rows of the wave (lane l: floats 256 i + 4 l ..
// + 3, head 4 i + l / 16, dims 4 (l % 16) ..), K and V as one (lanes with bit
// 4 clear: K dims 4 (l % 16) ..; set: V).
struct FoldRaw {
  f32x4 q0[kFoldMaxSplits], q1[kFoldMaxSplits], kv[kFoldMaxSplits];
};

// Every load issued at once, no branch between them (the sums come later, so
// the caller can issue its first KV blocks before it waits).
__device__ __forceinline__ void fold_issue(const AttnArgs& a, int b, int g, int lane, FoldRaw& f) {
  const PartView& pv = a.qkv;
  const int QD = a.n_q_heads * kD, G = 8;
  const int q0 = g * G * kD, kc = QD + g * kD, vc = QD + a.n_kv_heads * kD + g * kD;
  const float* row = pv.part + (long long)b * pv.ld;
  const long long ss = (long long)pv.rows * pv.ld;
  const int ckv = ((lane & 16) ? vc : kc) + 4 * (lane & 15);
#pragma unroll
  for (int s = 0; s < kFoldMaxSplits; ++s) {
    const float* p = row + min(s, pv.S - 1) * ss;
    f.q0[s] = *reinterpret_cast<const f32x4*>(p + q0 + 4 * lane);
    f.q1[s] = *reinterpret_cast<const f32x4*>(p + q0 + 256 + 4 * lane);
    f.kv[s] = *reinterpret_cast<const f32x4*>(p + ckv);
  }
}

// The split sum of the finish kernel, which takes a bound of 1, 2 or 4 splits
// and adds +0 for each split past S: with 3 splits one +0 (it turns a -0 sum
// into +0), otherwise none.
__device__ __forceinline__ f32x4 fold_sum(const f32x4 (&v)[kFoldMaxSplits], int S) {
  static_assert(kFoldMaxSplits == 4, "the finish's bounds for 1 to 4 splits are 1, 2, 4, 4");
  f32x4 acc = v[0];
#pragma unroll
  for (int s = 1; s < kFoldMaxSplits; ++s) acc = s < S ? acc + v[s] : acc;
  return S == 3 ? acc + f32x4{0.f, 0.f, 0.f, 0.f} : acc;
}

// Sums, bf16 rounding, and the moves to the lanes that use the values: q to
// the MFMA layout (lane (hl, q4): head hl's dims 32 h + 8 q4 .. + 7, the
// 4-dim chunks c = 8 h + 2 q4 + k of row hl / 4 at lane 16 (hl % 4) + c; the
// padding heads' lanes get 0); K the same dims in every lane; V dim
// d = 16 dt + lane % 16 in every lane (element d % 4 of chunk d / 4 at lane
// 16 + d / 4).
__device__ __forceinline__ void fold_make(const FoldRaw& f, int S, int lane, QRegs<DT_BF16>& qr, u32x4 (&kn)[2],
                                          uint32_t (&vn)[4]) {
  const int hl = lane & 15, q4 = lane >> 4;
  const f32x4 qs0 = fold_sum(f.q0, S), qs1 = fold_sum(f.q1, S), kvs = fold_sum(f.kv, S);
  const uint32_t qd00 = pack_bf16x2(qs0[0], qs0[1]), qd01 = pack_bf16x2(qs0[2], qs0[3]);
  const uint32_t qd10 = pack_bf16x2(qs1[0], qs1[1]), qd11 = pack_bf16x2(qs1[2], qs1[3]);
  const uint32_t kvd0 = pack_bf16x2(kvs[0], kvs[1]), kvd1 = pack_bf16x2(kvs[2], kvs[3]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t w[4], kw4[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = 8 * h + 2 * q4 + k, src = 16 * (hl & 3) + c;
      const uint32_t a0 = __shfl(qd00, src, 64), a1 = __shfl(qd01, src, 64);
      const uint32_t b0 = __shfl(qd10, src, 64), b1 = __shfl(qd11, src, 64);
      w[2 * k] = hl < 4 ? a0 : b0;
      w[2 * k + 1] = hl < 4 ? a1 : b1;
      kw4[2 * k] = __shfl(kvd0, c, 64);
      kw4[2 * k + 1] = __shfl(kvd1, c, 64);
    }
    qr.q[h] = hl < 8 ? u32x4{w[0], w[1], w[2], w[3]} : u32x4{0u, 0u, 0u, 0u};
    kn[h] = u32x4{kw4[0], kw4[1], kw4[2], kw4[3]};
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d = 16 * dt + (lane & 15), src = 16 + (d >> 2);
    const uint32_t a0 = __shfl(kvd0, src, 64), a1 = __shfl(kvd1, src, 64);
    const uint32_t wv = (d & 2) ? a1 : a0;
    vn[dt] = (d & 1) ? (wv >> 16) : (wv & 0xffffu);
  }
}

// The append of the new K row and V column at cache slot `slot` of a region
// (the cache is written through the region pointers it is read from): the
// lanes that hold the slot's K row and V entries store them.
__device__ __forceinline__ void fold_append(const char* kreg, const char* vreg, int slot, const u32x4 (&kn)[2],
                                            const uint32_t (&vn)[4], int lane) {
  const int s32 = slot & 31, q4 = lane >> 4;
  char* kw = const_cast<char*>(kreg);
  uint16_t* vw = (uint16_t*)const_cast<char*>(vreg);
  if ((lane & 15) == (s32 & 15)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) st16(kw + k_offset(slot, 32 * h + 8 * q4, 32) * 2, kn[h]);
  }
  if (q4 == ((s32 & 15) >> 2)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      vw[(long long)(slot >> 5) * 32 * kD + (16 * dt + (lane & 15)) * 32 + v_slot(s32)] = (uint16_t)vn[dt];
  }
}

// The new token's K row and V column of one window (bf16), patched into the
// registers of the block that holds its ring slot s32 (slot % 32): lanes with
// lane % 16 == s32 % 16 hold that slot's K row (tile s32 / 16) as dims
// 32 h + 8 (lane / 16) .. + 7; lanes with lane / 16 == (s32 % 16) / 4 hold its
// V entries, bf16 element v_slot(s32) % 8 of each d tile (d = 16 dt + lane % 16).
__device__ __forceinline__ void patch_new_slot(BlockRegs<DT_BF16>& br, const u32x4 (&kn)[2], const uint32_t (&vn)[4],
                                               int s32, int lane) {
  // value selects and masks only: a conditional store to a register array
  // element would be turned into an indexed store through scratch memory
  const int p16 = lane & 15, q4 = lane >> 4;
  const bool krow = p16 == (s32 & 15);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bool take = krow && (s32 >> 4) == t;
#pragma unroll
    for (int h = 0; h < 2; ++h) br.k[t][h] = take ? kn[h] : br.k[t][h];
  }
  const bool vcol = q4 == ((s32 & 15) >> 2);
  const int e = v_slot(s32) & 7;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const uint32_t sel = vcol && (e >> 1) == ww ? ((e & 1) ? 0xffff0000u : 0x0000ffffu) : 0u;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint32_t ins = (e & 1) ? (vn[dt] << 16) : vn[dt];
      br.v[dt][ww] = (br.v[dt][ww] & ~sel) | (ins & sel);
    }
  }
}

// Blocks [p0, p1) of the window of (token b, KV group g): the 4 waves stream
// their blocks, merge their states in wave order through LDS and write the
// output (pdst null: the piece is the whole window) or the piece's partial,
// [G][D + 2] floats at pdst. Every thread of the workgroup calls it; it ends
// with a barrier, so the LDS may be reused at once.
template <int KVT>
__device__ __forceinline__ void attn_piece_body(const AttnArgs& a, AttnLds& s, const KvLoc& loc, int b, int g, int p0,
                                                int p1, float* pdst, int G, int tid, int lane, int wave) {
  constexpr int esz = KVT == DT_BF16 ? 2 : 4;
  const char* kreg = (const char*)a.k_cache + loc.base * esz;
  const char* vreg = (const char*)a.v_cache + loc.base * esz;

  // query fragment: head (lane & 15) of this group
  const int hl = lane & 15, q4 = lane >> 4;
  const bool hvalid = hl < G;
  const char* qrow = (const char*)a.q + ((long long)b * a.n_q_heads + g * G + (hvalid ? hl : 0)) * kD * esz;
  QRegs<KVT> qr;
  if constexpr (KVT == DT_BF16) {
#pragma unroll
    for (int h = 0; h < 2; ++h) qr.q[h] = hvalid ? ld16(qrow + (32 * h + 8 * q4) * 2) : u32x4{0u, 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) qr.q[cc] = hvalid ? ld16(qrow + (16 * cc + 4 * q4) * 4) : u32x4{0u, 0u, 0u, 0u};
  }

  // this wave's blocks are blk0 + 4i, i < nbw
  const int blk0 = p0 + wave;
  const int nbw = p1 > blk0 ? (p1 - blk0 + 3) / 4 : 0;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nbw > 0) {
    // A ring of kRing register sets: a set is consumed, then refilled with
    // the block kRing steps ahead, so kRing - 1 blocks of loads stay in flight
    // while one is multiplied. The rounds are straight-line (scheduling
    // barriers keep each refill behind its consumer); a block index past this
    // wave's last block is clamped for the load and never attended.
    const int last = blk0 + 4 * (nbw - 1);
    BlockRegs<KVT> rb[kRing];
#pragma unroll
    for (int r = 0; r < kRing; ++r) load_block<KVT>(rb[r], kreg, vreg, min(blk0 + 4 * r, last), lane, kStreamKV);
    int i = 0;
    for (; i + kRing < nbw; i += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        attend<KVT>(rb[r], qr, blk0 + 4 * (i + r), loc.n_valid, a.scale_log2, m_run, l_run, acc, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_block<KVT>(rb[r], kreg, vreg, min(blk0 + 4 * (i + r + kRing), last), lane, kStreamKV);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int r = 0; r < kRing; ++r)
      if (i + r < nbw) attend<KVT>(rb[r], qr, blk0 + 4 * (i + r), loc.n_valid, a.scale_log2, m_run, l_run, acc, lane);
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // wave states -> LDS (O^T: lane holds d = 16 dt + 4 q4 + r of head hl)
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) s.o[wave][16 * dt + 4 * q4 + r][hl] = acc[dt][r];
  if (q4 == 0) {
    s.m[wave][hl] = m_run;
    s.l[wave][hl] = l_run;
  }
  __syncthreads();

  // merge the 4 waves (fixed order); thread -> (head, d) pairs
  const int GD = G * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i;
    if (idx >= GD) continue;
    const int h = idx >> 6, d = idx & 63;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s.m[w][h]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s.m[w][h];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      l += f * s.l[w][h];
      o += f * s.o[w][d][h];
    }
    if (pdst == nullptr) {
      // the whole window was in this piece: finish with the sink here
      const int hq = g * G + h;
      const float sink = a.sinks[hq] * kLog2e;
      const float MM = fmaxf(M, sink);
      const float f = M == -INFINITY ? 0.f : exp2f(M - MM);
      const float Z = exp2f(sink - MM) + f * l;
      const float out = f * o / Z;
      const long long oi = o_index(a, b, hq, d);
      if constexpr (KVT == DT_BF16) ((uint16_t*)a.o)[oi] = f32_to_bf16(out);
      else ((float*)a.o)[oi] = out;
    } else {
      float* pp = pdst + h * (kD + 2);
      pp[d] = o;
      if (d == 0) {
        pp[kD] = M;
        pp[kD + 1] = l;
      }
    }
  }
  __syncthreads();
}

// Workgroup = (chunk c, KV group g, token b).
template <int KVT, int KIND>
__global__ __launch_bounds__(256, SPA_ATTN_MINB) void k_attn(AttnArgs a) {
  __shared__ AttnLds s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar control flow
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int seq = a.tok0 + b;
  const int G = a.n_q_heads / a.n_kv_heads;
  if (a.tspan && tid == 0 && c == 0 && g == 0 && b == 0) a.tspan[0] = wall_clock64();   // first dispatched
  const KvLoc loc = kv_locate(a, seq, g, KIND);
  if (!loc.ok) {
    if (c == 0 && tid == 0 && a.err) atomicOr(a.err, ERR_KV_LEN);
    return;
  }
  const int n_chunks = (loc.n_valid + a.chunk - 1) / a.chunk;
  if (n_chunks > a.max_chunks) {   // kv_len above the planned maximum: refuse, never read past the plan
    if (c == 0 && tid == 0 && a.err) atomicOr(a.err, ERR_KV_LEN);
    return;
  }
  if (c >= n_chunks) return;
  // chunk c of n_chunks: an equal share of the window's blocks (at most
  // chunk / 32 of them), so no chunk is a short remainder
  const int nblk = (loc.n_valid + 31) / 32;
  float* pdst = n_chunks == 1 ? nullptr
                              : a.part + ((((long long)b * a.n_kv_heads + g) * a.max_chunks + c) * G) * (kD + 2);
  attn_piece_body<KVT>(a, s, loc, b, g, c * nblk / n_chunks, (c + 1) * nblk / n_chunks, pdst, G, tid, lane, wave);
  if (a.tspan) {   // uniform branch: every wave of the workgroup reaches it
    const int j = (c + (g + b * gridDim.y) * gridDim.x) & 15;
    if (tid == 0) atomicMax(a.tspan + 8 * (j + 1), (unsigned long long)wall_clock64());
  }
}

// Full layers, launches of up to kDealMaxTok (1,024) tokens. The launch's windows are
// laid end to end on one line of 32-position blocks, in (token, KV head)
// order, T blocks in all, and the line is cut into V equal ranges
// (v T / V .. (v + 1) T / V; V = a.deal_v, the same for every CU pool of the
// device, or T when T is smaller). A range's pieces of windows are computed
// like k_attn's chunks; a window inside one range is finished here, and a
// piece of a window that a range boundary cuts goes to partial slot
// (range + window index), which k_attn_merge combines in range order. The
// resident workgroup w of the stream's pool takes ranges w, w + W, ...: all
// ranges are the same work, so no CU is left with a long window while others
// idle. What a range computes depends on the launch's lengths and V only,
// never on W, so every schedule computes the same bits. Workgroup 0 also
// writes, per window, its first range and piece count for the merge
// (deal_tab).
// TPT: tokens per thread of the prologue (launches of up to 256 TPT tokens;
// the per-token tables in LDS are sized for them).
template <int KVT, int TPT>
__global__ __launch_bounds__(256, SPA_ATTN_MINB) void k_attn_dealt(AttnArgs a) {
  constexpr int NT = 256 * TPT;
  __shared__ AttnLds s;
  __shared__ long long s_first[NT + 1];   // first block of token t's windows on the line
  __shared__ long long s_off[NT];
  __shared__ int s_len[NT], s_cap[NT], s_nb[NT];   // s_nb: blocks per window, 0 if refused
  __shared__ int s_wsum[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.n_q_heads / a.n_kv_heads, Hkv = a.n_kv_heads;
  const int n = a.n_tok;   // 1 .. NT: tokens TPT tid .. TPT tid + TPT - 1 per thread
  if (a.tspan && tid == 0 && blockIdx.x == 0) a.tspan[0] = wall_clock64();   // first dispatched
  int nbv[TPT], local = 0;   // the thread's block counts and their sum
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int t = tid * TPT + u;
    nbv[u] = 0;
    if (t < n) {
      const int seq = a.tok0 + t;
      const int L = a.kv_len[seq], cap = a.kv_cap[seq];
      const long long off = a.kv_off[seq];
      const bool ok = L >= 1 && L <= cap;
      if (!ok && blockIdx.x == 0 && a.err) atomicOr(a.err, ERR_KV_LEN);   // refused: no blocks, reported once
      nbv[u] = ok ? (L + 31) / 32 : 0;
      s_len[t] = L;
      s_cap[t] = cap;
      s_off[t] = off;
      s_nb[t] = nbv[u];
    }
    local += nbv[u];
  }
  // exclusive prefix of the per-token block counts in token order: the
  // thread's own tokens, a wave scan of the thread sums, then the wave sums
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < wave; ++w2) before += s_wsum[w2];
  int run = before + incl - local;
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int t = tid * TPT + u;
    if (t < n) s_first[t] = (long long)run * Hkv;
    run += nbv[u];
  }
  if (tid == 0) s_first[n] = (long long)(s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3]) * Hkv;
  __syncthreads();
  const long long T = s_first[n];
  const int V = (int)min((long long)a.deal_v, T);
  // range holding block x: the largest v with v T / V <= x
  auto range_of = [&](long long x) { return (int)(((x + 1) * V - 1) / T); };
  if (blockIdx.x == 0) {
    for (int j = tid; j < n * Hkv; j += 256) {
      const int t = j / Hkv, g = j - t * Hkv, nbt = s_nb[t];
      int first = 0, cnt = 0;
      if (nbt > 0) {
        const long long ws = s_first[t] + (long long)g * nbt;
        first = range_of(ws);
        cnt = range_of(ws + nbt - 1) - first + 1;
      }
      a.deal_tab[2 * j] = first;
      a.deal_tab[2 * j + 1] = cnt;
    }
  }
  const int W = gridDim.x, w = blockIdx.x;
  for (int v = w; v < V; v += W) {
    const long long lo = (long long)v * T / V, hi = (long long)(v + 1) * T / V;
    int t = 0, t1 = n - 1;   // token holding block lo: the largest t with s_first[t] <= lo (it has blocks)
    while (t < t1) {
      const int mid = (t + t1 + 1) >> 1;
      if (s_first[mid] <= lo) t = mid;
      else t1 = mid - 1;
    }
    int nbt = s_nb[t];
    int g = (int)((lo - s_first[t]) / nbt);
    long long ws = s_first[t] + (long long)g * nbt;   // the window's first block on the line
    long long x = lo;
    for (;;) {
      const int p0 = (int)(x - ws), p1 = (int)(min(hi, ws + nbt) - ws);
      const int j = t * Hkv + g;
      KvLoc loc;
      loc.base = (s_off[t] * Hkv + (long long)g * s_cap[t]) * kD;
      loc.n_valid = s_len[t];
      loc.ok = true;
      float* pdst = (p0 == 0 && p1 == nbt) ? nullptr : a.part + (long long)(v + j) * G * (kD + 2);
      attn_piece_body<KVT>(a, s, loc, t, g, p0, p1, pdst, G, tid, lane, wave);
      x = ws + p1;
      if (x >= hi) break;
      if (++g == Hkv) {   // the next token with blocks (one exists: x < hi <= T)
        g = 0;
        do ++t; while (t < n && s_nb[t] == 0);
        if (t >= n) break;
        nbt = s_nb[t];
      }
      ws = s_first[t] + (long long)g * nbt;
    }
  }
  if (a.tspan && tid == 0) atomicMax(a.tspan + 8 * ((w & 15) + 1), (unsigned long long)wall_clock64());
}

// Sliding layers at large batches: one wave per window (token b, KV head g),
// four windows per workgroup. The wave streams the window's blocks through
// its register ring and finishes with the sink itself: no piece merge through
// LDS and no barrier, so the workgroup's fixed costs are shared by four
// windows. A lane holds head (lane & 15) and dims 16 dt + 4 (lane >> 4) + r,
// so each lane stores four runs of four outputs.
// With a.qkv set (bf16) the QKV finish is folded in (fold_issue ..
// fold_append): the new K/V sit at ring slot (L - 1) % W.
template <int KVT>
__global__ __launch_bounds__(256, SPA_ATTN_MINB) void k_attn_wave(AttnArgs a) {
  constexpr int esz = KVT == DT_BF16 ? 2 : 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.n_q_heads / a.n_kv_heads, Hkv = a.n_kv_heads;
  if (a.tspan && tid == 0 && blockIdx.x == 0) a.tspan[0] = wall_clock64();   // first dispatched
  const int j = blockIdx.x * 4 + wave;   // wave-uniform; the kernel has no workgroup barrier
  if (j < a.n_tok * Hkv) {
    const int b = j / Hkv, g = j - b * Hkv;
    const KvLoc loc = kv_locate(a, a.tok0 + b, g, KV_RING);
    if (!loc.ok) {
      if (lane == 0 && g == 0 && a.err) atomicOr(a.err, ERR_KV_LEN);
    } else {
      const char* kreg = (const char*)a.k_cache + loc.base * esz;
      const char* vreg = (const char*)a.v_cache + loc.base * esz;
      const int hl = lane & 15, q4 = lane >> 4;
      const bool hvalid = hl < G;
      const char* qrow = (const char*)a.q + ((long long)b * a.n_q_heads + g * G + (hvalid ? hl : 0)) * kD * esz;
      QRegs<KVT> qr;
      u32x4 kn[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
      uint32_t vn[4] = {0u, 0u, 0u, 0u};
      int sblk = -1, s32 = 0;
      const int nb = (loc.n_valid + 31) / 32;
      // blocks 0 .. nb-1 through a ring of kRing register sets (a block past
      // the last is clamped for the load and never attended)
      BlockRegs<KVT> rb[kRing];
      const bool fold = KVT == DT_BF16 && a.qkv.part != nullptr;
      if (fold) {
        if constexpr (KVT == DT_BF16) {
          // the ring's first loads go out with the finish's loads, ahead of
          // their sums and of the append's stores
          FoldRaw fr;
          fold_issue(a, b, g, lane, fr);
#pragma unroll
          for (int r = 0; r < kRing; ++r) load_block<KVT>(rb[r], kreg, vreg, min(r, nb - 1), lane, kStreamKV);
          const int slot = (a.kv_len[a.tok0 + b] - 1) % a.window;   // L >= 1 (loc.ok)
          sblk = slot >> 5;
          s32 = slot & 31;
          fold_make(fr, a.qkv.S, lane, qr, kn, vn);
          fold_append(kreg, vreg, slot, kn, vn, lane);
        }
      } else {
        if constexpr (KVT == DT_BF16) {
#pragma unroll
          for (int h = 0; h < 2; ++h) qr.q[h] = hvalid ? ld16(qrow + (32 * h + 8 * q4) * 2) : u32x4{0u, 0u, 0u, 0u};
        } else {
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
            qr.q[cc] = hvalid ? ld16(qrow + (16 * cc + 4 * q4) * 4) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < kRing; ++r) load_block<KVT>(rb[r], kreg, vreg, min(r, nb - 1), lane, kStreamKV);
      }
      const float sink = a.sinks[g * G + (hvalid ? hl : 0)] * kLog2e;
      float m_run = -INFINITY, l_run = 0.f;
      f32x4 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      int i = 0;
      for (; i + kRing < nb; i += kRing) {
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
          if constexpr (KVT == DT_BF16)
            if (i + r == sblk) patch_new_slot(rb[r], kn, vn, s32, lane);   // sblk = -1 unless folded
          attend<KVT>(rb[r], qr, i + r, loc.n_valid, a.scale_log2, m_run, l_run, acc, lane);
          __builtin_amdgcn_sched_barrier(0);
          load_block<KVT>(rb[r], kreg, vreg, min(i + r + kRing, nb - 1), lane, kStreamKV);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int r = 0; r < kRing; ++r)
        if (i + r < nb) {
          if constexpr (KVT == DT_BF16)
            if (i + r == sblk) patch_new_slot(rb[r], kn, vn, s32, lane);
          attend<KVT>(rb[r], qr, i + r, loc.n_valid, a.scale_log2, m_run, l_run, acc, lane);
        }
      l_run += __shfl_xor(l_run, 16, 64);
      l_run += __shfl_xor(l_run, 32, 64);
      if (hvalid) {
        const float MM = fmaxf(m_run, sink);
        const float f = m_run == -INFINITY ? 0.f : exp2f(m_run - MM);
        const float Z = exp2f(sink - MM) + f * l_run;
        const float fz = f / Z;
        const int hq = g * G + hl;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const long long oi = o_index(a, b, hq, 16 * dt + 4 * q4);   // four consecutive outputs
          if constexpr (KVT == DT_BF16) {
            *reinterpret_cast<uint2*>((uint16_t*)a.o + oi) =
                uint2{pack_bf16x2(acc[dt][0] * fz, acc[dt][1] * fz), pack_bf16x2(acc[dt][2] * fz, acc[dt][3] * fz)};
          } else {
            *reinterpret_cast<f32x4*>((float*)a.o + oi) =
                f32x4{acc[dt][0] * fz, acc[dt][1] * fz, acc[dt][2] * fz, acc[dt][3] * fz};
          }
        }
      }
    }
  }
  if (a.tspan && lane == 0) atomicMax(a.tspan + 8 * ((blockIdx.x & 15) + 1), (unsigned long long)wall_clock64());
}

// Merge the piece partials of one (sequence, KV head) in window order with the
// sink: M = max(sink, m_c), Z = 2^(sink-M) + sum l_c 2^(m_c-M), o = sum o_c 2^(m_c-M) / Z.
// k_attn's chunks sit at [b][g][chunk]; k_attn_dealt's pieces of window j at
// the consecutive slots first + j + i, i < count, from deal_tab.
template <int KVT>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int seq = a.tok0 + b;
  const int G = a.n_q_heads / a.n_kv_heads;
  int n_chunks;
  long long pbase;
  if (a.deal_v > 0) {
    const int j = b * a.n_kv_heads + g;
    n_chunks = a.deal_tab[2 * j + 1];
    if (n_chunks <= 1) return;
    pbase = (long long)(a.deal_tab[2 * j] + j) * G * (kD + 2);
  } else {
    const KvLoc loc = kv_locate(a, seq, g, a.kv_kind);
    if (!loc.ok) return;
    n_chunks = (loc.n_valid + a.chunk - 1) / a.chunk;
    if (n_chunks <= 1 || n_chunks > a.max_chunks) return;
    pbase = (((long long)b * a.n_kv_heads + g) * a.max_chunks) * G * (kD + 2);
  }
  const long long cstride = (long long)G * (kD + 2);
  constexpr int UF = 8;   // up to UF chunks and 2 (head, d) pairs per thread: one pass, every load first
  if (n_chunks <= UF && G * kD <= 512) {
    float mv[2][UF], lv[2][UF], ov[2][UF], sk[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = min(tid + 256 * j, G * kD - 1);
      const int h = idx >> 6, d = idx & 63;
      sk[j] = a.sinks[g * G + h];
      const float* pp = a.part + pbase + (long long)h * (kD + 2);
#pragma unroll
      for (int i = 0; i < UF; ++i) {
        const float* q = pp + min(i, n_chunks - 1) * cstride;
        mv[j][i] = q[kD];
        lv[j][i] = q[kD + 1];
        ov[j][i] = q[d];
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + 256 * j;
      if (idx >= G * kD) continue;
      const int h = idx >> 6, d = idx & 63;
      const float sink = sk[j] * kLog2e;
      float M = sink;
#pragma unroll
      for (int i = 0; i < UF; ++i) M = fmaxf(M, mv[j][i]);   // clamped repeats do not change a max
      float Z = exp2f(sink - M), o = 0.f;
#pragma unroll
      for (int i = 0; i < UF; ++i) {
        if (i >= n_chunks) break;
        const float f = mv[j][i] == -INFINITY ? 0.f : exp2f(mv[j][i] - M);
        Z += f * lv[j][i];
        o += f * ov[j][i];
      }
      const float out = o / Z;
      const long long oi = o_index(a, b, g * G + h, d);
      if constexpr (KVT == DT_BF16) ((uint16_t*)a.o)[oi] = f32_to_bf16(out);
      else ((float*)a.o)[oi] = out;
    }
    return;
  }
  constexpr int U = 16;   // chunk states loaded together (clamped, masked)
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx >> 6, d = idx & 63;
    const int hq = g * G + h;
    const float sink = a.sinks[hq] * kLog2e;
    const float* pp = a.part + pbase + (long long)h * (kD + 2);
    float M = sink;
    for (int c0 = 0; c0 < n_chunks; c0 += U) {
      float mv[U];
#pragma unroll
      for (int i = 0; i < U; ++i) mv[i] = pp[min(c0 + i, n_chunks - 1) * cstride + kD];
#pragma unroll
      for (int i = 0; i < U; ++i) M = fmaxf(M, mv[i]);   // clamped repeats do not change a max
    }
    float Z = exp2f(sink - M), o = 0.f;
    for (int c0 = 0; c0 < n_chunks; c0 += U) {
      float mv[U], lv[U], ov[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float* q = pp + min(c0 + i, n_chunks - 1) * cstride;
        mv[i] = q[kD];
        lv[i] = q[kD + 1];
        ov[i] = q[d];
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if (c0 + i >= n_chunks) break;
        const float f = mv[i] == -INFINITY ? 0.f : exp2f(mv[i] - M);
        Z += f * lv[i];
        o += f * ov[i];
      }
    }
    const float out = o / Z;
    const long long oi = o_index(a, b, hq, d);
    if constexpr (KVT == DT_BF16) ((uint16_t*)a.o)[oi] = f32_to_bf16(out);
    else ((float*)a.o)[oi] = out;
  }
}

template <int KVT, int KIND>
static void launch_attn_t(const AttnArgs& a, dim3 grid, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  if (start || stop)
    hipExtLaunchKernelGGL((k_attn<KVT, KIND>), grid, dim3(256), 0, st, start, stop, 0, a);
  else
    hipLaunchKernelGGL((k_attn<KVT, KIND>), grid, dim3(256), 0, st, a);
}

template <int KVT, int TPT>
static void launch_dealt_tpt(const AttnArgs& a, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  if (start || stop)
    hipExtLaunchKernelGGL((k_attn_dealt<KVT, TPT>), dim3(a.deal_wgs), dim3(256), 0, st, start, stop, 0, a);
  else
    hipLaunchKernelGGL((k_attn_dealt<KVT, TPT>), dim3(a.deal_wgs), dim3(256), 0, st, a);
}

// up to 256 tokens: one token per prologue thread and the smaller tables
template <int KVT>
static void launch_dealt_t(const AttnArgs& a, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  static_assert(kDealMaxTok == 4 * 256, "the prologue instances cover 256 and 1024 tokens");
  if (a.n_tok <= 256) launch_dealt_tpt<KVT, 1>(a, st, start, stop);
  else launch_dealt_tpt<KVT, 4>(a, st, start, stop);
}

template <int KVT>
static void launch_wave_t(const AttnArgs& a, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  const dim3 grid((a.n_tok * a.n_kv_heads + 3) / 4);
  if (start || stop)
    hipExtLaunchKernelGGL(k_attn_wave<KVT>, grid, dim3(256), 0, st, start, stop, 0, a);
  else
    hipLaunchKernelGGL(k_attn_wave<KVT>, grid, dim3(256), 0, st, a);
}

// The shapes the folded QKV finish handles (fold_issue .. fold_append).
static bool fold_args_ok(const AttnArgs& a) {
  return a.kv_dtype == DT_BF16 && a.head_dim == kD && a.n_q_heads == 8 * a.n_kv_heads && a.qkv.S >= 1 &&
         a.qkv.S <= kFoldMaxSplits && a.qkv.rows >= a.n_tok && a.qkv.ld % 4 == 0 &&
         a.qkv.ld >= (a.n_q_heads + 2 * a.n_kv_heads) * kD;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  if (a.wave_windows) {
    if (a.kv_kind != KV_RING || a.deal_wgs > 0 || a.n_q_heads / a.n_kv_heads > 16) return hipErrorInvalidValue;
    if (a.qkv.part && !fold_args_ok(a)) return hipErrorInvalidValue;
    if (a.kv_dtype == DT_BF16) launch_wave_t<DT_BF16>(a, st, start, stop);
    else launch_wave_t<DT_F32>(a, st, start, stop);
    return hipGetLastError();
  }
  if (a.deal_wgs > 0 && a.kv_kind == KV_PACKED) {
    if (a.n_tok < 1 || a.n_tok > kDealMaxTok || a.deal_v < 1 || a.deal_v > kDealMaxRanges || !a.deal_tab)
      return hipErrorInvalidValue;
    if (a.qkv.part) return hipErrorInvalidValue;   // the even split takes q and appended K/V
    if (a.kv_dtype == DT_BF16) launch_dealt_t<DT_BF16>(a, st, start, stop);
    else launch_dealt_t<DT_F32>(a, st, start, stop);
    return hipGetLastError();
  }
  if (a.qkv.part) return hipErrorInvalidValue;   // the chunk grid takes q and appended K/V
  dim3 grid(a.max_chunks, a.n_kv_heads, a.n_tok);
  if (a.kv_dtype == DT_BF16) {
    if (a.kv_kind == KV_PACKED) launch_attn_t<DT_BF16, KV_PACKED>(a, grid, st, start, stop);
    else launch_attn_t<DT_BF16, KV_RING>(a, grid, st, start, stop);
  } else {
    if (a.kv_kind == KV_PACKED) launch_attn_t<DT_F32, KV_PACKED>(a, grid, st, start, stop);
    else launch_attn_t<DT_F32, KV_RING>(a, grid, st, start, stop);
  }
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.n_kv_heads, a.n_tok);
  if (a.kv_dtype == DT_BF16) hipLaunchKernelGGL(k_attn_merge<DT_BF16>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_attn_merge<DT_F32>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace spa
