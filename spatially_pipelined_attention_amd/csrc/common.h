// Shared device helpers for the gfx950 kernels (CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (NaN stays NaN): the gfx950 packed
// conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)pack_bf16x2(f, 0.f); }

// Barrier that orders LDS only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// A lane's partner value inside its 16-lane row by DPP (a VALU operand
// modifier, no LDS round trip): lane ^ 1, lane ^ 2 (quad permutes), the
// mirror inside each half row (i <-> 7 - i) and inside the row
// (i <-> 15 - i). Each is an involution, so after the four steps every lane
// of a row has combined the same 16 values (exact for max).
template <int STEP>
__device__ __forceinline__ int dpp_partner(int x) {
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  return __builtin_amdgcn_update_dpp(0, x, ctrl, 0xF, 0xF, false);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_partner<0>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_partner<1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_partner<2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_partner<3>(__float_as_int(v))));
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

template <typename T, typename S>
__device__ __forceinline__ T bitcast(S s) {
  static_assert(sizeof(T) == sizeof(S), "bitcast size");
  return __builtin_bit_cast(T, s);
}

// Element (r, c) of a split-K product: its S partials (split stride rows *
// ld floats) summed in split order; SM >= S is a compile-time bound, and the
// padding terms add +0. part_sum4 does the same for columns c .. c + 3 (c a
// multiple of 4, ld too), element by element in the same order.
template <int SM, class View>
__device__ __forceinline__ float part_sum(const View& pv, int r, int c) {
  const float* p = pv.part + (long long)r * pv.ld + c;
  const long long sstride = (long long)pv.rows * pv.ld;
  float v[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) v[s] = p[min(s, pv.S - 1) * sstride];
  float acc = v[0];
#pragma unroll
  for (int s = 1; s < SM; ++s) acc += s < pv.S ? v[s] : 0.f;
  return acc;
}

template <int SM, class View>
__device__ __forceinline__ f32x4 part_sum4(const View& pv, int r, int c) {
  const float* p = pv.part + (long long)r * pv.ld + c;
  const long long sstride = (long long)pv.rows * pv.ld;
  f32x4 v[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) v[s] = *reinterpret_cast<const f32x4*>(p + min(s, pv.S - 1) * sstride);
  f32x4 acc = v[0];
#pragma unroll
  for (int s = 1; s < SM; ++s) acc += s < pv.S ? v[s] : f32x4{0.f, 0.f, 0.f, 0.f};
  return acc;
}

// Position p of a 32-position KV block -> storage slot inside the block's
// d-major V tile. Two 16-position halves are interleaved in runs of four so
// that one lane's eight MFMA k-slots (positions 4q..4q+3 of both halves) are
// one contiguous 16-byte run.
// K element (slot, d) of a cache region (D = 64): 32-slot blocks, each split
// into 64-byte column groups of kpe = 64 / element-size dims stored slot by
// slot, so 16 slots of one column group are 1 KB of contiguous memory.
__host__ __device__ __forceinline__ long long k_offset(int slot, int d, int kpe) {
  return (long long)(slot >> 5) * 32 * 64 + (d / kpe) * 32 * kpe + (slot & 31) * kpe + d % kpe;
}

__host__ __device__ __forceinline__ int v_slot(int p) {
  return 8 * ((p & 15) >> 2) + 4 * (p >> 4) + (p & 3);
}

// OCP E4M3 value of a finite float already in [-448, 448]: round to nearest
// even on 3 mantissa bits (quantum 2^-9 below 2^-6).
__device__ __forceinline__ uint8_t f32_to_e4m3(float f) {
  uint32_t u = __float_as_uint(f);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  float a = fabsf(f);
  if (a >= 448.0f) return sign | 0x7Eu;
  int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;   // a == 0 gives -127
  if (e < -6) e = -6;
  float q = __uint_as_float((uint32_t)(e - 3 + 127) << 23);  // 2^(e-3)
  float n = __builtin_rintf(a / q);                            // ties to even
  float v = n * q;
  if (v >= 448.0f) return sign | 0x7Eu;
  if (v == 0.0f) return sign;
  int ev = (int)((__float_as_uint(v) >> 23) & 0xff) - 127;
  if (ev < -6) return sign | (uint8_t)(int)(v * 512.0f);      // subnormal: mant * 2^-9
  int mant = (int)(v / __uint_as_float((uint32_t)(ev - 3 + 127) << 23)) - 8;
  return sign | (uint8_t)(((ev + 7) << 3) | mant);
}

}  // namespace spa
