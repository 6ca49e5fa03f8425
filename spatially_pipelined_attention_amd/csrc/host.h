// Host-side internals shared by the C ABI translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "kernels.h"
#include "spa.h"

struct spa_ctx {
  int device = 0;
  int n_cus = 0;
  int n_xcd = 8;
  int wall_khz = 100000;   // device wall clock (wall_clock64) rate
  hipDeviceProp_t prop{};
};

namespace spa {

void set_error(const std::string& msg);
spa_status fail(spa_status code, const std::string& msg);
spa_status hip_fail(hipError_t e, const char* what);

#define SPA_HIP(call)                                   \
  do {                                                  \
    hipError_t _e = (call);                             \
    if (_e != hipSuccess) return ::spa::hip_fail(_e, #call); \
  } while (0)

// Kernel classes (timing hooks and split heuristics).
enum KClass : int {
  KC_ATTN_FULL = 0, KC_ATTN_SLIDING = 1, KC_QKV = 2, KC_OPROJ = 3,
  KC_ROUTER = 4, KC_GATEUP = 5, KC_DOWN = 6, KC_COMBINE = 7, KC_COMM = 8, KC_COUNT = 9
};

#ifndef SPA_ATTN_CHUNK
#define SPA_ATTN_CHUNK 512
#endif
constexpr int kAttnChunk = SPA_ATTN_CHUNK;   // cached positions per attention workgroup (multiple of 128)

// Byte layout of one microbatch slot of the workspace.
struct SlotLayout {
  size_t xn, q, o, h, hn_f32, hn_bf16, hn8, hn8_scale, logits;
  size_t topk_idx, topk_w, offsets, row_tok, row_slot, inv;
  size_t xe_perm, xe_perm_scale, z, z8, z8_scale, y, attn_part, gemm_part;
  size_t comm;          // receive buffer of the virtual communication endpoints
  size_t bytes;
};

// Workspace header: the error word and the launch counters, cleared at the
// start of every run (words 32..63: MoE-head hand-offs, 64..127: routing)
constexpr int kHeaderWords = 128;

struct WsLayout {
  size_t err;           // int32 error word (shared by all slots)
  size_t slot0;         // first slot
  size_t slot_bytes;
  int n_slots;
  int n_tok;            // tokens per slot
  int max_chunks;
  size_t total;
  SlotLayout s;
};

struct GemmPlan {
  int n_tiles, n_groups, S, rb_stride, ks, epi;
  int tile_cols, blk_rows, part_rows, part_ld;
};

spa_status validate_model(const spa_model_desc* m);
bool comm_enabled(const spa_model_desc* m);
// Launch one virtual communication endpoint: copy copy_bytes (a multiple of
// 16) src -> dst; the launch lasts latency_us + bytes / gbps.
spa_status launch_comm(spa_ctx* ctx, const void* src, void* dst, size_t copy_bytes, size_t bytes, double latency_us,
                       double gbps, hipStream_t st);
WsLayout ws_layout(const spa_model_desc* m, int n_tok, int max_kv_len, int n_micro);
int max_chunks_for(int max_kv_len, const spa_model_desc* m);
GemmPlan plan_gemm(int kclass, const spa_model_desc* m, int n_tok, int n_cus);
// Decode attention with its scratch handed over (no workspace): bytes of
// chunk partials a call needs, the argument checks of spa_decode_attn, and
// the launch itself (SPA_EWORKSPACE when part_bytes is too small).
size_t attn_scratch_bytes(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int n_tok,
                          int* max_chunks_out);
spa_status check_decode_attn_args(const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0, int n_tok,
                                  const void* q, const void* o_out);
spa_status decode_attn_on_scratch(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b,
                                  int tok0, int n_tok, const void* q, void* o, float* part, size_t part_bytes,
                                  int32_t* err_word, bool clear_err, hipStream_t st);
// Looks up this device's copy of the no-allocation scratch array (once per
// device; the device must be current). Called by spa_init.
spa_status noalloc_bind_device(int device);

// CUs a stream's kernels run on: the pool's count for a CU-masked pool
// stream (registered by the pool), `fallback` for any other stream.
void register_stream_cus(hipStream_t st, int n_cus);
void unregister_stream_cus(hipStream_t st);
int stream_cus(hipStream_t st, int fallback);

// Per-slot device pointers resolved from a workspace base.
struct Slot {
  char* base;
  int* err;
  unsigned* head_ctr;   // two zeroed counters for the MoE-head launch's hand-offs (null: none)
  unsigned* route_ctr;  // zeroed arrival counter of the routing launch (null: none)
  void* xn;
  void* q;
  void* o;
  float* h;
  float* hn_f32;
  uint16_t* hn_bf16;
  uint8_t* hn8;
  float* hn8_scale;
  float* logits;
  spa_route_bufs route;
  void* z;
  uint8_t* z8;
  float* z8_scale;
  void* xe_perm;
  float* xe_perm_scale;
  float* y;
  float* attn_part;
  float* gemm_part;
  void* comm;
};

Slot slot_ptrs(const WsLayout& L, void* ws, int slot);

// Timing hook: called around each kernel launch of a class (may be null).
struct TimingHook {
  int cls = -1;
  std::vector<hipEvent_t>* evs = nullptr;   // pairs (start, stop)
  std::vector<hipEvent_t>* pool = nullptr;  // free events
  // device-clock spans (attention kernels): launch i owns
  // span[i * kSpanWords, (i + 1) * kSpanWords); null when the launches are
  // timed by events instead
  unsigned long long* span = nullptr;
  int* span_used = nullptr;
  int span_cap = 0;
};

// The layer's pieces on one slot (tokens [tok0, tok0+n_tok)); enqueue on st.
// with_router: segment A also routes (output projection through the gather);
// fuse_head: that part may run as the one-launch MoE head.
spa_status run_segment_a(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int layer_index,
                         const spa_layer* next, const spa_batch* b, int tok0, int n_tok, const WsLayout& W,
                         const Slot& s, bool with_router, bool first_layer, hipStream_t st, TimingHook* th,
                         bool fuse_head = false);
spa_status run_segment_b(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int layer_index,
                         const spa_layer* next, const spa_batch* b, int tok0, int n_tok, const WsLayout& W,
                         const Slot& s, bool with_router, hipStream_t st, TimingHook* th);
// The layer around its attention (for the Macro cut): before (first layer:
// RMSNorm of x; QKV, KV append), the attention, after (output projection to
// combine).
spa_status run_layer_before_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b,
                                 int tok0, int n_tok, const Slot& s, bool first_layer, hipStream_t st, TimingHook* th);
spa_status run_layer_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0,
                          int n_tok, const WsLayout& W, const Slot& s, hipStream_t st, TimingHook* th);
spa_status run_layer_after_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int layer_index,
                                const spa_layer* next, const spa_batch* b, int tok0, int n_tok, const WsLayout& W,
                                const Slot& s, hipStream_t st, TimingHook* th, bool fuse_head = false);
spa_status clear_errors(void* ws, hipStream_t st);

}  // namespace spa
