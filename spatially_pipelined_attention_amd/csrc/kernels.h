// Launch interfaces of the gfx950 kernels (host <-> device argument blocks).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

// Storage type codes shared with the C ABI (spa_dtype).
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

enum XMode : int { XM_RAW = 0, XM_NORM = 1 };
enum Epi : int { EPI_QKV = 0, EPI_RESID_SS = 1, EPI_SWIGLU = 2, EPI_STORE = 3, EPI_ROUTER = 4 };
enum KvKind : int { KV_RING = 0, KV_PACKED = 1 };

// device-side error bits (workspace error word)
enum : int { ERR_KV_LEN = 1, ERR_ROUTE = 2 };

struct GemmArgs {
  // weights: group g's matrix starts at W + g * w_gstride elements, rows of K
  const void* W;
  long long w_gstride;
  int K;
  int N;                    // output columns (SwiGLU: inter)
  const float* w_scale;     // E4M3: per W row scale, group stride ws_gstride
  long long ws_gstride;
  int n_tiles;              // 64-wide output column tiles
  int n_groups;
  const int* group_off;     // [n_groups+1] or null (one group of n_rows)
  int n_rows;
  int S;                    // split-K factor
  // X
  const void* X;
  int x_ld;
  const int* row_src;       // X row of each output row (null: identity)
  const float* ss;          // row sum-of-squares partials [ss_tiles][ss_ld]
  int ss_tiles;
  int ss_ld;
  const float* gamma;
  float eps;
  float inv_h;
  const float* x_scale;     // E4M3 X: per X row scale
  // split-K workspace
  float* part;
  int* ctr;
  int rb_stride;
  // outputs
  void* out;
  int out_ld;
  int out_dtype;
  const float* resid;
  int resid_ld;
  float* ss_out;
  int ss_out_ld;
  int inter;
  // QKV epilogue
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  int kv_dtype;
  int kv_kind;
  void* k_cache;
  void* v_cache;
  const int* kv_len;
  const long long* kv_off;
  const int* kv_cap;
  int window;
  int tok0;
  int* err;
  // router epilogue
  int* done_ctr;
  int top_k;
  int n_resident;
  int* topk_idx;
  float* topk_w;
  int* topk_rec;
  int* route_off;
  int* row_tok;
  int* row_slot;
  int* inv;
};

hipError_t launch_gemm(int wt, int xm, int epi, const GemmArgs& a, hipStream_t st);

struct AttnArgs {
  const void* q;            // [n_tok][Hq][D] (bf16 or f32 = kv dtype)
  const void* k_cache;
  const void* v_cache;
  int kv_dtype;
  int kv_kind;
  const int* kv_len;        // indexed by sequence (tok0 + b)
  const long long* kv_off;
  const int* kv_cap;
  int window;
  int tok0;
  int n_tok;
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  const float* sinks;       // [Hq]
  float scale_log2;         // softmax scale * log2(e)
  int chunk;                // positions per workgroup (multiple of 128)
  int max_chunks;
  float* part;              // [n_tok][Hkv][max_chunks][G][D+2]
  int* ctr;                 // [n_tok][Hkv]
  void* o;                  // [n_tok][Hq*D] (bf16 or f32 = kv dtype)
  int* err;
  int stream_kv;            // non-temporal KV loads
};

hipError_t launch_attn(const AttnArgs& a, hipStream_t st);

struct CombineArgs {
  const float* h;           // [n_tok][H]
  const float* y;           // [R][H] expert outputs (rows in dispatch order)
  const float* w;           // [n_tok][k]
  const int* inv;           // [n_tok][k]
  int k;
  int n_tok;
  int H;
  float* x_out;             // [n_tok][H]
  float* ss_out;            // [H/64][ss_ld]
  int ss_ld;
};

hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// rows of an fp32 matrix -> (x * rstd * gamma) quantised to per-row power-of-two-scaled E4M3
struct QuantArgs {
  const float* x;
  int x_ld;
  int n_rows;
  int n_cols;
  const int* row_src;       // optional gather
  const int* n_rows_dev;    // optional device row count (<= n_rows)
  const float* ss;          // optional RMSNorm (with gamma); null: plain rows
  int ss_tiles;
  int ss_ld;
  const float* gamma;
  float eps;
  float inv_h;
  uint8_t* codes;           // [n_rows][n_cols]
  float* scales;            // [n_rows]
};

hipError_t launch_quant_e4m3(const QuantArgs& a, hipStream_t st);

hipError_t launch_fill_i32(int* p, long long n, int v, hipStream_t st);

struct KvIoArgs {
  void* k_cache;
  void* v_cache;
  int kv_dtype;
  int kv_kind;
  const long long* kv_off;
  const int* kv_cap;
  int window;
  int n_kv_heads;
  int head_dim;
  const int* seq;           // [n]
  const int* pos;           // [n]
  int n;
  int n_seq;                // sequences in the batch (seq[] must be below)
  void* k_rows;             // [n][Hkv][D]
  void* v_rows;
  int write;                // 1: rows -> cache, 0: cache -> rows
};

hipError_t launch_kv_io(const KvIoArgs& a, hipStream_t st);

// hardware placement probe: each workgroup records its XCC / SE / CU ids
hipError_t launch_probe(unsigned* out, int n_blocks, int spin, hipStream_t st);

int gemm_lds_bytes();

}  // namespace spa
