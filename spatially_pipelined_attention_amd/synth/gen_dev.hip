// Seeded synthetic-input generator, device side (HIP, gfx950).
//
// Twin of gen_host.c: the same counter-based hash (the SplitMix64 output mix
// of Steele, Lea and Flood, OOPSLA 2014, over a Weyl sequence) and the same
// Irwin-Hall(4) normal draw, so device-filled inputs are bit-identical to the
// host generator's. Holds no arithmetic of the decode layer; used only to
// fill large synthetic inputs in HBM without a host round trip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SPA_GOLDEN 0x9E3779B97F4A7C15ULL

__device__ __forceinline__ uint64_t spa_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float spa_draw(uint64_t key, uint64_t i, float scale) {
  uint64_t h = spa_mix64(key + (i + 1ULL) * SPA_GOLDEN);
  uint32_t s = (uint32_t)(h & 0xFFFFu) + (uint32_t)((h >> 16) & 0xFFFFu) +
               (uint32_t)((h >> 32) & 0xFFFFu) + (uint32_t)(h >> 48);
  // one IEEE multiply of an exact integer: no contraction possible
  return __fmul_rn((float)((int32_t)s - 131070), scale);
}

__device__ __forceinline__ uint16_t spa_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void k_gen_normal_f32(float* out, int64_t n, uint64_t key, int64_t i0, float scale) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n;
       j += (int64_t)gridDim.x * blockDim.x)
    out[j] = spa_draw(key, (uint64_t)(i0 + j), scale);
}

__global__ void k_gen_normal_bf16(uint16_t* out, int64_t n, uint64_t key, int64_t i0, float scale) {
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n;
       j += (int64_t)gridDim.x * blockDim.x)
    out[j] = spa_bf16_rne(spa_draw(key, (uint64_t)(i0 + j), scale));
}

// Rows of a [n_rows][row_len] bf16 tensor whose element (r, c) is draw index
// base[r] + c: lets a caller fill many independent runs (one per sequence and
// head, say) in one launch.
__global__ void k_gen_rows_bf16(uint16_t* out, int64_t n_rows, int64_t row_len,
                                const int64_t* base, uint64_t key, float scale) {
  int64_t total = n_rows * row_len;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < total;
       j += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = j / row_len, c = j - r * row_len;
    out[j] = spa_bf16_rne(spa_draw(key, (uint64_t)(base[r] + c), scale));
  }
}

__global__ void k_gen_rows_f32(float* out, int64_t n_rows, int64_t row_len,
                               const int64_t* base, uint64_t key, float scale) {
  int64_t total = n_rows * row_len;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < total;
       j += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = j / row_len, c = j - r * row_len;
    out[j] = spa_draw(key, (uint64_t)(base[r] + c), scale);
  }
}

static int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

extern "C" {

// All entry points: device output pointer, element count, stream key, first
// draw index, fp32 scale, HIP stream (0 = null stream). Returns hipError_t.
int spa_gen_dev_normal_f32(float* out, int64_t n, uint64_t key, int64_t i0, float scale, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_gen_normal_f32, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     out, n, key, i0, scale);
  return (int)hipGetLastError();
}

int spa_gen_dev_normal_bf16(uint16_t* out, int64_t n, uint64_t key, int64_t i0, float scale, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_gen_normal_bf16, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     out, n, key, i0, scale);
  return (int)hipGetLastError();
}

int spa_gen_dev_rows_bf16(uint16_t* out, int64_t n_rows, int64_t row_len, const int64_t* base_dev,
                          uint64_t key, float scale, void* stream) {
  if (n_rows <= 0 || row_len <= 0) return 0;
  hipLaunchKernelGGL(k_gen_rows_bf16, dim3(grid_for(n_rows * row_len)), dim3(256), 0,
                     (hipStream_t)stream, out, n_rows, row_len, base_dev, key, scale);
  return (int)hipGetLastError();
}

int spa_gen_dev_rows_f32(float* out, int64_t n_rows, int64_t row_len, const int64_t* base_dev,
                         uint64_t key, float scale, void* stream) {
  if (n_rows <= 0 || row_len <= 0) return 0;
  hipLaunchKernelGGL(k_gen_rows_f32, dim3(grid_for(n_rows * row_len)), dim3(256), 0,
                     (hipStream_t)stream, out, n_rows, row_len, base_dev, key, scale);
  return (int)hipGetLastError();
}

}  // extern "C"
