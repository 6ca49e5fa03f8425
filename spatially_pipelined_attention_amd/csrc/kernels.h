// Launch interfaces of the gfx950 kernels (host <-> device argument blocks).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

// Storage type codes shared with the C ABI (spa_dtype).
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

enum Epi : int { EPI_PARTIAL = 0, EPI_SWIGLU = 1, EPI_STORE = 2 };
enum KvKind : int { KV_RING = 0, KV_PACKED = 1 };

// device-side error bits (workspace error word)
enum : int { ERR_KV_LEN = 1, ERR_HANDOFF = 2 };

// Split-K partial products: fp32 [split][rows][ld]; rows are token rows of a
// dense product or dispatch rows of a grouped one, ld the padded column count.
struct PartView {
  const float* part;
  int S;
  int rows;
  int ld;
};

struct GemmArgs {
  const void* W;            // group g's matrix at W + g * w_gstride elements, [rows][K]
  long long w_gstride;
  int K;
  int N;                    // output columns (SwiGLU: inter)
  const float* w_scale;     // E4M3: per W row scale, group stride ws_gstride
  long long ws_gstride;
  int n_tiles;              // output column tiles of tile_cols (SwiGLU: half gate, half up)
  int tile_cols;            // 16 (fp32 router), 32, 48, 64, 96, or 128 (the LDS-tiled kernel)
  int blk_rows;             // rows per row block (16, 32, 48, 64, 80 or 128)
  int n_groups;
  const int* group_off;     // [n_groups+1] or null (one group of n_rows)
  int n_rows;
  int S;                    // split-K factor
  const void* X;            // rows of K elements in the weight's MFMA input type
  long long x_rstride;      // bytes between rows (row-major: K * esz; k-step-major: 64)
  long long x_kstride;      // bytes between 64-byte k-steps (row-major: 64; k-step-major: rows * 64)
  const int* row_src;       // X row of each output row (null: identity)
  const float* x_scale;     // E4M3 X: per X row scale
  float* part;              // EPI_PARTIAL output [S][part_rows][part_ld]
  int part_rows;
  int part_ld;
  int rb_stride;            // row-block slots in the grid (grouped: upper bound on non-empty blocks)
  void* out;                // EPI_SWIGLU / EPI_STORE output
  int out_ld;
  int out_kmajor_rows;      // SwiGLU: > 0 writes z k-step-major over this many rows (else row-major, out_ld)
  int out_dtype;
  int inter;
};

hipError_t launch_gemm(int wt, int epi, const GemmArgs& a, hipStream_t st);
// The 128-row x 128-column LDS-tiled variant (gemm_big.hip): blk_rows 128,
// tile_cols 128 (SwiGLU: 64 outputs), split-K for partials only.
hipError_t launch_gemm_big(int wt, int epi, const GemmArgs& a, hipStream_t st);

// q + KV append from the QKV partials, one workgroup per token row.
struct QkvFinishArgs {
  PartView pv;
  int n_tok;
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  void* q_out;              // [n_tok][Hq*D], kv dtype
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
  float rope_theta;         // > 0: rotary embedding of q and k at position L-1
};
hipError_t launch_qkv_finish(const QkvFinishArgs& a, hipStream_t st);

// h = x + o Wo^T (from partials); hn = RMSNorm(h) * gamma in fp32, bf16 and
// optionally per-row power-of-two-scaled E4M3.
struct OprojFinishArgs {
  PartView pv;
  int n_tok;
  int H;
  const float* x;
  float* h_out;
  const float* gamma;
  float eps;
  float* hn_f32;
  uint16_t* hn_bf16;        // optional
  uint8_t* hn_e4m3;         // optional
  float* hn_scale;
};
hipError_t launch_oproj_finish(const OprojFinishArgs& a, hipStream_t st);

// Router logits (from partials) -> top-k -> softmax weights -> permutation. One workgroup.
struct RouteArgs {
  PartView pv;
  int n_tok;
  int E;
  int k;
  int E_res;
  float* logits;            // [n_tok][E]
  int* topk_idx;
  float* topk_w;
  int* topk_rec;            // optional
  int* offsets;
  int* row_tok;
  int* row_slot;
  int* inv;
  // optional gather of the expert input rows into dispatch order (k-step-major)
  const void* gsrc;         // [n_tok][gK] row-major, element size gesz
  int gK;
  int gesz;
  void* gdst;               // [gK*gesz/64][n_tok*k][64 bytes]
  const float* gsrc_scale;  // E4M3: per source row
  float* gdst_scale;        // E4M3: per dispatch row
  // zeroed arrival counter (no gather only): the last top-k workgroup to
  // finish runs the permutation and clears it again; null: a second launch
  unsigned* arrive;
};
// top-k, then the permutation (and the gather when gsrc is set)
hipError_t launch_route(const RouteArgs& a, hipStream_t st);

// The MoE head (output projection finish, router GEMV, top-k, permutation and
// gather) as one persistent launch of G workgroups of 1024 threads with
// device hand-offs between its phases (misc.hip). ctr: two zeroed counters,
// cleared again by the launch itself; err: device error word (ERR_HANDOFF).
struct MoeHeadArgs {
  OprojFinishArgs of;       // phase 0
  GemmArgs router;          // phase 1: the router product (fp32 16-column tiles, split partials)
  int n_router_tiles;       // its tiles: n_tiles * rb_stride * S
  RouteArgs ra;             // phases 2 and 3 (ra.pv: the router partials)
  unsigned* ctr;
  int* err;
};
// splits of the output projection and the router, rows per router block
bool moe_head_supported(int oproj_splits, int router_splits, int router_blk_rows);
hipError_t launch_moe_head(const MoeHeadArgs& a, int G, hipStream_t st);

// x_out = h + sum_s w[s] * y[inv[s]]; optionally xn = RMSNorm(x_out) * gamma
// for the next projection. y is plain [R][H] or split partials of the
// expert-down product (rows grouped by expert with group offsets).
struct CombineArgs {
  const float* h;
  const float* y;           // plain y (or null)
  PartView ypv;             // partial y (dispatch rows) when y == null
  const int* y_group_off;   // [y_n_groups + 1]: dispatch rows in use = y_group_off[y_n_groups]
  int y_n_groups;
  const float* w;
  const int* inv;
  int k;
  int n_tok;
  int H;
  float* x_out;
  const float* gamma_next;  // null: no normalised output
  float eps;
  void* xn_out;
  int xn_dtype;
  int xn_kmajor_rows;       // > 0: xn is k-step-major over this many rows (64-byte k-steps)
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);
// out (a.x_out)[r] = split sum of dispatch row r of the grouped partial y (a.ypv)
hipError_t launch_part_rows(const CombineArgs& a, int max_rows, hipStream_t st);

struct AttnArgs {
  const void* q;            // [n_tok][Hq][D] (kv dtype)
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
  float* part;              // k_attn: [n_tok][Hkv][max_chunks][G][D+2]; k_attn_dealt: [deal_v + n_tok*Hkv][G][D+2]
  void* o;                  // [n_tok][Hq*D] (kv dtype)
  int* err;
  int stream_kv;            // non-temporal KV loads
  int o_kmajor_rows;        // > 0: o is k-step-major over this many rows (64-byte k-steps)
  // optional [kSpanWords]: this launch's span on the device wall clock. The
  // first workgroup stores its start in word 0; every workgroup takes the
  // atomic max of its end into word 8 (j + 1), j = its linear index mod 16
  // (spread over 16 lines, so the atomics do not queue on one address).
  // The caller presets the words to zero.
  unsigned long long* tspan;
  // > 0: full layers as an even split of the launch's blocks into deal_v
  // ranges, taken by this many resident workgroups (k_attn_dealt); 0: one
  // workgroup per chunk (k_attn)
  int deal_wgs;
  int deal_v;               // ranges of the even split (the same for every pool of the device)
  int* deal_tab;            // [n_tok * Hkv][2]: first range and piece count of each window
  // 1 (sliding layers): one wave per window, four windows per workgroup
  // (k_attn_wave); 0: a window's blocks spread over the four waves
  int wave_windows;
  // k_attn_wave, bf16 KV, 8 query heads per KV head: the QKV split partials
  // (at most kFoldMaxSplits) of the launch's tokens (row b
  // = token b; q at columns [0, Hq D), K at Hq D + g D, V at (Hq + Hkv) D + g D).
  // The kernel then sums q and the new K/V itself and appends K/V (the QKV
  // finish folded in); part null: q is given and K/V are already appended.
  PartView qkv;
};
constexpr int kSpanWords = 136;
constexpr int kFoldMaxSplits = 4;   // QKV splits the one-wave-per-window attention sums itself
constexpr int kDealMaxTok = 1024;   // tokens per launch of the dealt kernel (one or four per prologue thread)
#ifndef SPA_DEAL_RANGES_PER_CU
#define SPA_DEAL_RANGES_PER_CU 2
#endif
constexpr int kDealRangesPerCu = SPA_DEAL_RANGES_PER_CU;   // ranges of the split per CU of the device
constexpr int kDealMaxRanges = 2048;   // upper bound of deal_v (workspace sizing)
#ifndef SPA_DEAL_WGS_PER_CU
#define SPA_DEAL_WGS_PER_CU 2
#endif
constexpr int kDealWgsPerCu = SPA_DEAL_WGS_PER_CU;   // resident workgroups per CU it deals to
// start/stop (optional): events recorded around the launch
hipError_t launch_attn(const AttnArgs& a, hipStream_t st, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// merge of the chunk partials of multi-chunk sequences (single-chunk ones are final already)
hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t st);

// fp32 rows -> bf16 rows or per-row power-of-two-scaled E4M3 (expert inputs).
// kmajor_rows > 0: input and output are k-step-major over that many rows
// (element (r, c) of a 64-byte k-step layout sits at ((c / ks) * rows + r) * ks + c % ks).
struct CvtArgs {
  const float* x;
  int n_rows;
  int n_cols;
  int dtype;                // DT_BF16 or DT_E4M3
  void* out;
  float* scales;            // E4M3
  int kmajor_rows;
  int n_cus;                // device CUs: picks the workgroup size
};
hipError_t launch_cvt_rows(const CvtArgs& a, hipStream_t st);

hipError_t launch_fill_i32(int* p, long long n, int v, hipStream_t st);
// Folds n recorded launch spans (kSpanWords words each, as the attention
// kernels write them) into acc[0] += sum of (latest end - start) ticks and
// acc[1] += the number of spans with a start (one workgroup, in span order),
// then clears the n spans for the next launches.
hipError_t launch_span_fold(unsigned long long* spans, int n, unsigned long long* acc, hipStream_t st);
// Kernel attributes the launches rely on; call before any stream capture.
hipError_t init_kernel_attributes();

// Virtual communication endpoint: copy n16 16-byte words src -> dst, then
// keep every workgroup resident until `ticks` device wall-clock ticks after
// it started (a collective's modelled duration).
hipError_t launch_virtual_comm(const void* src, void* dst, long long n16, unsigned long long ticks, hipStream_t st);

// Row-major [n_mats][N][K] (element size esz, K * esz a multiple of 64) ->
// panels [n_mats][ceil(N/16)][K*esz/64][16 rows][64 bytes]; rows past N are zero.
hipError_t launch_pack_panels(const void* src, void* dst, int n_mats, int N, int K, int esz, hipStream_t st);

// dst k-step-major [K*esz/64][R][64 bytes] <- rows src[row_src[r]] of a
// row-major [*][K] source; optional per-row scales gathered alongside.
hipError_t launch_gather_kmajor(const void* src, const int* row_src, int R, int K, int esz, void* dst,
                                const float* src_scale, float* dst_scale, hipStream_t st);

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

bool gemm_blk_rows_ok(int rows);

}  // namespace spa
