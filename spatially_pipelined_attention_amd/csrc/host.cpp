// Host side of the C ABI: validation, workspace carving, operator launches,
// the layer's two segments, single-layer and temporal execution.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "host.h"

namespace spa {

static thread_local std::string g_err;

void set_error(const std::string& msg) { g_err = msg; }
spa_status fail(spa_status code, const std::string& msg) {
  g_err = msg;
  return code;
}
spa_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return SPA_EHIP;
}

static int ks_of(int dt) { return dt == DT_BF16 ? 32 : (dt == DT_F32 ? 16 : 64); }
static int esz_of(int dt) { return dt == DT_BF16 ? 2 : (dt == DT_F32 ? 4 : 1); }
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

spa_status validate_model(const spa_model_desc* m) {
  if (!m) return fail(SPA_EINVAL, "model descriptor is NULL");
  if (m->head_dim != 64) return fail(SPA_EUNSUPPORTED, "head_dim must be 64");
  if (m->n_q_heads <= 0 || m->n_kv_heads <= 0 || m->n_q_heads % m->n_kv_heads)
    return fail(SPA_EINVAL, "n_q_heads must be a positive multiple of n_kv_heads");
  if (m->n_q_heads / m->n_kv_heads > 16) return fail(SPA_EUNSUPPORTED, "more than 16 query heads per KV head");
  if (m->hidden <= 0 || m->hidden % 64) return fail(SPA_EINVAL, "hidden must be a positive multiple of 64");
  if (m->inter <= 0 || m->inter % 32) return fail(SPA_EINVAL, "inter must be a positive multiple of 32");
  if (m->window <= 0 || m->window % 32) return fail(SPA_EINVAL, "window must be a positive multiple of 32");
  if (m->n_experts < 1 || m->n_experts > 256) return fail(SPA_EUNSUPPORTED, "n_experts must be in [1, 256]");
  if (m->top_k < 1 || m->top_k > 8 || m->top_k > m->n_experts) return fail(SPA_EINVAL, "top_k must be in [1, min(E, 8)]");
  if (m->n_resident < 1 || m->n_resident > m->n_experts) return fail(SPA_EINVAL, "n_resident must be in [1, E]");
  if (m->n_layers < 1) return fail(SPA_EINVAL, "n_layers must be >= 1");
  if (!(m->eps >= 0.f)) return fail(SPA_EINVAL, "eps must be >= 0");
  if (m->dense_dtype != SPA_F32 && m->dense_dtype != SPA_BF16) return fail(SPA_EUNSUPPORTED, "dense_dtype must be F32 or BF16");
  if (m->kv_dtype != m->dense_dtype) return fail(SPA_EUNSUPPORTED, "kv_dtype must equal dense_dtype");
  if (m->expert_dtype != SPA_F32 && m->expert_dtype != SPA_BF16 && m->expert_dtype != SPA_E4M3)
    return fail(SPA_EINVAL, "bad expert_dtype");
  if (m->expert_dtype == SPA_E4M3 && m->dense_dtype != SPA_BF16)
    return fail(SPA_EUNSUPPORTED, "E4M3 experts need BF16 dense weights");
  const int ksd = ks_of(m->dense_dtype), kse = ks_of(m->expert_dtype);
  if (m->hidden % ksd || (m->n_q_heads * m->head_dim) % ksd)
    return fail(SPA_EUNSUPPORTED, "hidden and Hq*D must be multiples of the dense k-step");
  if (m->hidden % kse || m->inter % kse)
    return fail(SPA_EUNSUPPORTED, "hidden and inter must be multiples of the expert k-step");
  if (m->hidden % 16) return fail(SPA_EUNSUPPORTED, "hidden must be a multiple of 16 (router)");
  return SPA_OK;
}

int max_chunks_for(int max_kv_len, const spa_model_desc* m) {
  int l = std::max(max_kv_len, m->window);
  return (l + kAttnChunk - 1) / kAttnChunk;
}

GemmPlan plan_gemm(int kc, const spa_model_desc* m, int n_tok, int n_cus) {
  GemmPlan p{};
  int N = 0, K = 0, groups = 1, rows = n_tok;
  switch (kc) {
    case KC_QKV: N = (m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim; K = m->hidden; p.ks = ks_of(m->dense_dtype);
      p.n_tiles = N / 64; break;
    case KC_OPROJ: N = m->hidden; K = m->n_q_heads * m->head_dim; p.ks = ks_of(m->dense_dtype); p.n_tiles = N / 64; break;
    case KC_ROUTER: N = m->n_experts; K = m->hidden; p.ks = 16; p.n_tiles = (N + 63) / 64; break;
    case KC_GATEUP: N = m->inter; K = m->hidden; p.ks = ks_of(m->expert_dtype); p.n_tiles = N / 32;
      groups = m->n_resident; rows = n_tok * m->top_k; break;
    case KC_DOWN: N = m->hidden; K = m->inter; p.ks = ks_of(m->expert_dtype); p.n_tiles = N / 64;
      groups = m->n_resident; rows = n_tok * m->top_k; break;
    default: break;
  }
  p.n_groups = groups;
  p.rb_stride = std::max(1, (rows + 63) / 64);
  const int nks = K / p.ks;
  const int target = std::max(256, (n_cus * 5) / 4);
  int S = (target + p.n_tiles * groups - 1) / (p.n_tiles * groups);
  S = std::min(S, std::max(1, nks / 8));
  p.S = std::max(1, S);
  return p;
}

WsLayout ws_layout(const spa_model_desc* m, int n_tok, int max_kv_len, int n_micro) {
  WsLayout L{};
  const int H = m->hidden, Hq = m->n_q_heads, Hkv = m->n_kv_heads, D = m->head_dim;
  const int G = Hq / Hkv, k = m->top_k, E = m->n_experts, Er = m->n_resident, I = m->inter;
  const int R = n_tok * k;
  const int nbh = H / 64;
  const size_t kv_esz = esz_of(m->kv_dtype);
  const bool fp8 = m->expert_dtype == SPA_E4M3;
  L.n_slots = n_micro;
  L.n_tok = n_tok;
  L.max_chunks = max_chunks_for(max_kv_len, m);

  // counters of one slot
  size_t gemm_ctr_n = 0, gemm_part_n = 0;
  for (int kc : {KC_QKV, KC_OPROJ, KC_ROUTER, KC_GATEUP, KC_DOWN}) {
    GemmPlan p = plan_gemm(kc, m, n_tok, 1024);   // upper bound on S for any device
    size_t tiles = (size_t)p.n_groups * p.n_tiles * p.rb_stride;
    gemm_ctr_n = std::max(gemm_ctr_n, tiles);
  }
  // partials sized for the S actually used on this device are computed at
  // run time; reserve for the largest S any plan can give (nks / 8 bound)
  for (int kc : {KC_QKV, KC_OPROJ, KC_ROUTER, KC_GATEUP, KC_DOWN}) {
    GemmPlan p = plan_gemm(kc, m, n_tok, 1024);
    if (p.S > 1) gemm_part_n = std::max(gemm_part_n, (size_t)p.n_groups * p.n_tiles * p.rb_stride * p.S * 4096);
  }

  SlotLayout& s = L.s;
  size_t o = 0;
  // --- counters first (cleared together) ---
  s.attn_ctr = o; o = align256(o + (size_t)n_tok * Hkv * 4);
  s.gemm_ctr = o; o = align256(o + gemm_ctr_n * 5 * 4);   // one region per GEMM class
  s.done_ctr = o; o = align256(o + 64);
  const size_t ctr_bytes = o;
  // --- data ---
  s.ss_x = o; o = align256(o + (size_t)nbh * n_tok * 4);
  s.ss_h = o; o = align256(o + (size_t)nbh * n_tok * 4);
  s.q = o; o = align256(o + (size_t)n_tok * Hq * D * kv_esz);
  s.o = o; o = align256(o + (size_t)n_tok * Hq * D * kv_esz);
  s.h = o; o = align256(o + (size_t)n_tok * H * 4);
  s.logits = o; o = align256(o + (size_t)n_tok * E * 4);
  s.topk_idx = o; o = align256(o + (size_t)R * 4);
  s.topk_w = o; o = align256(o + (size_t)R * 4);
  s.offsets = o; o = align256(o + (size_t)(Er + 1) * 4);
  s.row_tok = o; o = align256(o + (size_t)R * 4);
  s.row_slot = o; o = align256(o + (size_t)R * 4);
  s.inv = o; o = align256(o + (size_t)R * 4);
  s.hq8 = o; o = align256(o + (fp8 ? (size_t)n_tok * H : 0));
  s.hq8_scale = o; o = align256(o + (fp8 ? (size_t)n_tok * 4 : 0));
  s.z = o; o = align256(o + (size_t)R * I * (m->expert_dtype == SPA_BF16 ? 2 : 4));
  s.z8 = o; o = align256(o + (fp8 ? (size_t)R * I : 0));
  s.z8_scale = o; o = align256(o + (fp8 ? (size_t)R * 4 : 0));
  s.y = o; o = align256(o + (size_t)R * H * 4);
  s.attn_part = o; o = align256(o + (size_t)n_tok * Hkv * L.max_chunks * G * (D + 2) * 4);
  s.gemm_part = o; o = align256(o + gemm_part_n * 4);
  s.bytes = o;

  L.err = 0;
  L.slot0 = 256;
  L.slot_bytes = s.bytes;
  L.total = L.slot0 + (size_t)n_micro * s.bytes;
  L.ctr_begin = 0;
  L.ctr_end = ctr_bytes;
  return L;
}

Slot slot_ptrs(const WsLayout& L, void* ws, int slot) {
  Slot s{};
  char* b = (char*)ws + L.slot0 + (size_t)slot * L.slot_bytes;
  const SlotLayout& o = L.s;
  s.base = b;
  s.err = (int*)((char*)ws + L.err);
  s.ss_x = (float*)(b + o.ss_x);
  s.ss_h = (float*)(b + o.ss_h);
  s.q = b + o.q;
  s.o = b + o.o;
  s.h = (float*)(b + o.h);
  s.logits = (float*)(b + o.logits);
  s.route.topk_idx = (int32_t*)(b + o.topk_idx);
  s.route.topk_w = (float*)(b + o.topk_w);
  s.route.offsets = (int32_t*)(b + o.offsets);
  s.route.row_tok = (int32_t*)(b + o.row_tok);
  s.route.row_slot = (int32_t*)(b + o.row_slot);
  s.route.inv = (int32_t*)(b + o.inv);
  s.hq8 = (uint8_t*)(b + o.hq8);
  s.hq8_scale = (float*)(b + o.hq8_scale);
  s.z = b + o.z;
  s.z8 = (uint8_t*)(b + o.z8);
  s.z8_scale = (float*)(b + o.z8_scale);
  s.y = (float*)(b + o.y);
  s.attn_part = (float*)(b + o.attn_part);
  s.gemm_part = (float*)(b + o.gemm_part);
  s.attn_ctr = (int*)(b + o.attn_ctr);
  s.gemm_ctr = (int*)(b + o.gemm_ctr);
  s.done_ctr = (int*)(b + o.done_ctr);
  return s;
}

spa_status clear_counters(const WsLayout& W, void* ws, hipStream_t st) {
  SPA_HIP(launch_fill_i32((int*)ws, 64, 0, st));   // error word + pad
  for (int i = 0; i < W.n_slots; ++i) {
    char* b = (char*)ws + W.slot0 + (size_t)i * W.slot_bytes;
    SPA_HIP(launch_fill_i32((int*)(b + W.ctr_begin), (long long)((W.ctr_end - W.ctr_begin) / 4), 0, st));
  }
  return SPA_OK;
}

static int gemm_ctr_region(int kc) {
  switch (kc) {
    case KC_QKV: return 0;
    case KC_OPROJ: return 1;
    case KC_ROUTER: return 2;
    case KC_GATEUP: return 3;
    default: return 4;
  }
}

// ---------------------------------------------------------------------------
// timing hook
// ---------------------------------------------------------------------------
struct HookScope {
  TimingHook* th;
  hipStream_t st;
  bool on;
  HookScope(TimingHook* t, int cls, hipStream_t s) : th(t), st(s), on(t && t->cls == cls && t->evs && t->pool) {
    if (on) th->evs->push_back(take());
    if (on) (void)hipEventRecord(th->evs->back(), st);
  }
  hipEvent_t take() {
    if (th->pool->empty()) {
      hipEvent_t e;
      (void)hipEventCreate(&e);
      return e;
    }
    hipEvent_t e = th->pool->back();
    th->pool->pop_back();
    return e;
  }
  ~HookScope() {
    if (on) {
      th->evs->push_back(take());
      (void)hipEventRecord(th->evs->back(), st);
    }
  }
};

// ---------------------------------------------------------------------------
// operators (explicit pointers; scratch from slot s)
// ---------------------------------------------------------------------------
static GemmArgs gemm_base(const GemmPlan& p, const Slot& s, int kc, int n_tok, const spa_model_desc* m) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.n_tiles = p.n_tiles;
  a.n_groups = p.n_groups;
  a.S = p.S;
  a.rb_stride = p.rb_stride;
  a.n_rows = n_tok;
  a.part = s.gemm_part;
  size_t region = 0;
  {
    // counter region per class: sized by the largest tile count of any class
    GemmPlan worst{};
    size_t mx = 0;
    for (int c : {KC_QKV, KC_OPROJ, KC_ROUTER, KC_GATEUP, KC_DOWN}) {
      worst = plan_gemm(c, m, n_tok, 1024);
      mx = std::max(mx, (size_t)worst.n_groups * worst.n_tiles * worst.rb_stride);
    }
    region = mx * gemm_ctr_region(kc);
  }
  a.ctr = s.gemm_ctr + region;
  a.err = s.err;
  a.eps = m->eps;
  a.inv_h = 1.0f / (float)m->hidden;
  return a;
}

static spa_status op_qkv(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0,
                         int n_tok, const float* ss_x, int ss_ld, void* q_out, const Slot& s, hipStream_t st,
                         TimingHook* th) {
  GemmPlan p = plan_gemm(KC_QKV, m, n_tok, ctx->n_cus);
  GemmArgs a = gemm_base(p, s, KC_QKV, n_tok, m);
  a.W = l->wqkv;
  a.K = m->hidden;
  a.N = (m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim;
  a.X = b->x + (size_t)tok0 * m->hidden;
  a.x_ld = m->hidden;
  a.ss = ss_x;
  a.ss_tiles = m->hidden / 64;
  a.ss_ld = ss_ld;
  a.gamma = l->gamma1;
  a.out = q_out;
  a.out_ld = m->n_q_heads * m->head_dim;
  a.out_dtype = m->kv_dtype;
  a.n_q_heads = m->n_q_heads;
  a.n_kv_heads = m->n_kv_heads;
  a.head_dim = m->head_dim;
  a.kv_dtype = m->kv_dtype;
  a.kv_kind = l->kind == SPA_FULL ? KV_PACKED : KV_RING;
  a.k_cache = l->k_cache;
  a.v_cache = l->v_cache;
  a.kv_len = b->kv_len;
  a.kv_off = (const long long*)b->kv_off;
  a.kv_cap = b->kv_cap;
  a.window = m->window;
  a.tok0 = tok0;
  HookScope hs(th, KC_QKV, st);
  SPA_HIP(launch_gemm(m->dense_dtype, XM_NORM, EPI_QKV, a, st));
  return SPA_OK;
}

static spa_status op_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0,
                          int n_tok, const void* q, void* o, const WsLayout& W, const Slot& s, hipStream_t st,
                          TimingHook* th) {
  (void)ctx;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k_cache = l->k_cache;
  a.v_cache = l->v_cache;
  a.kv_dtype = m->kv_dtype;
  a.kv_kind = l->kind == SPA_FULL ? KV_PACKED : KV_RING;
  a.kv_len = b->kv_len;
  a.kv_off = (const long long*)b->kv_off;
  a.kv_cap = b->kv_cap;
  a.window = m->window;
  a.tok0 = tok0;
  a.n_tok = n_tok;
  a.n_q_heads = m->n_q_heads;
  a.n_kv_heads = m->n_kv_heads;
  a.head_dim = m->head_dim;
  a.sinks = l->sinks;
  a.scale_log2 = (float)(1.0 / std::sqrt((double)m->head_dim) * 1.4426950408889634);
  a.chunk = kAttnChunk;
  a.max_chunks = l->kind == SPA_FULL ? W.max_chunks : (m->window + kAttnChunk - 1) / kAttnChunk;
  a.part = s.attn_part;
  a.ctr = s.attn_ctr;
  a.o = o;
  a.err = s.err;
  a.stream_kv = 1;
  HookScope hs(th, l->kind == SPA_FULL ? KC_ATTN_FULL : KC_ATTN_SLIDING, st);
  SPA_HIP(launch_attn(a, st));
  return SPA_OK;
}

static spa_status op_oproj(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* x, const void* o,
                           int n_tok, float* h, float* ss_h, int ss_ld, const Slot& s, hipStream_t st,
                           TimingHook* th) {
  GemmPlan p = plan_gemm(KC_OPROJ, m, n_tok, ctx->n_cus);
  GemmArgs a = gemm_base(p, s, KC_OPROJ, n_tok, m);
  a.W = l->wo;
  a.K = m->n_q_heads * m->head_dim;
  a.N = m->hidden;
  a.X = o;
  a.x_ld = m->n_q_heads * m->head_dim;
  a.out = h;
  a.out_ld = m->hidden;
  a.resid = x;
  a.resid_ld = m->hidden;
  a.ss_out = ss_h;
  a.ss_out_ld = ss_ld;
  HookScope hs(th, KC_OPROJ, st);
  SPA_HIP(launch_gemm(m->dense_dtype, XM_RAW, EPI_RESID_SS, a, st));
  return SPA_OK;
}

static spa_status op_route(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* h,
                           const float* ss_h, int ss_ld, int n_tok, float* logits, const spa_route_bufs& r,
                           int32_t* topk_rec, const Slot& s, hipStream_t st, TimingHook* th) {
  GemmPlan p = plan_gemm(KC_ROUTER, m, n_tok, ctx->n_cus);
  GemmArgs a = gemm_base(p, s, KC_ROUTER, n_tok, m);
  a.W = l->wr;
  a.K = m->hidden;
  a.N = m->n_experts;
  a.X = h;
  a.x_ld = m->hidden;
  a.ss = ss_h;
  a.ss_tiles = m->hidden / 64;
  a.ss_ld = ss_ld;
  a.gamma = l->gamma2;
  a.out = logits;
  a.out_ld = m->n_experts;
  a.done_ctr = s.done_ctr;
  a.top_k = m->top_k;
  a.n_resident = m->n_resident;
  a.topk_idx = r.topk_idx;
  a.topk_w = r.topk_w;
  a.topk_rec = topk_rec;
  a.route_off = r.offsets;
  a.row_tok = r.row_tok;
  a.row_slot = r.row_slot;
  a.inv = r.inv;
  HookScope hs(th, KC_ROUTER, st);
  SPA_HIP(launch_gemm(DT_F32, XM_NORM, EPI_ROUTER, a, st));
  return SPA_OK;
}

static spa_status op_expert(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* h,
                            const float* ss_h, int ss_ld, int n_tok, const spa_route_bufs& r, float* y, const Slot& s,
                            hipStream_t st, TimingHook* th) {
  const int H = m->hidden, I = m->inter, R = n_tok * m->top_k;
  const bool fp8 = m->expert_dtype == SPA_E4M3;
  if (fp8) {
    QuantArgs qa;
    memset(&qa, 0, sizeof(qa));
    qa.x = h;
    qa.x_ld = H;
    qa.n_rows = n_tok;
    qa.n_cols = H;
    qa.ss = ss_h;
    qa.ss_tiles = H / 64;
    qa.ss_ld = ss_ld;
    qa.gamma = l->gamma2;
    qa.eps = m->eps;
    qa.inv_h = 1.0f / (float)H;
    qa.codes = s.hq8;
    qa.scales = s.hq8_scale;
    HookScope hs(th, KC_GATEUP, st);
    SPA_HIP(launch_quant_e4m3(qa, st));
  }
  {
    GemmPlan p = plan_gemm(KC_GATEUP, m, n_tok, ctx->n_cus);
    GemmArgs a = gemm_base(p, s, KC_GATEUP, n_tok, m);
    a.W = l->wgu;
    a.w_gstride = (long long)2 * I * H;
    a.w_scale = l->wgu_scale;
    a.ws_gstride = 2 * I;
    a.K = H;
    a.N = I;
    a.inter = I;
    a.group_off = r.offsets;
    a.row_src = r.row_tok;
    a.out = s.z;
    a.out_ld = I;
    a.out_dtype = m->expert_dtype == SPA_BF16 ? DT_BF16 : DT_F32;
    if (fp8) {
      a.X = s.hq8;
      a.x_ld = H;
      a.x_scale = s.hq8_scale;
    } else {
      a.X = h;
      a.x_ld = H;
      a.ss = ss_h;
      a.ss_tiles = H / 64;
      a.ss_ld = ss_ld;
      a.gamma = l->gamma2;
    }
    HookScope hs(th, KC_GATEUP, st);
    SPA_HIP(launch_gemm(m->expert_dtype, fp8 ? XM_RAW : XM_NORM, EPI_SWIGLU, a, st));
  }
  if (fp8) {
    QuantArgs qa;
    memset(&qa, 0, sizeof(qa));
    qa.x = (const float*)s.z;
    qa.x_ld = I;
    qa.n_rows = R;
    qa.n_cols = I;
    qa.codes = s.z8;
    qa.scales = s.z8_scale;
    HookScope hs(th, KC_DOWN, st);
    SPA_HIP(launch_quant_e4m3(qa, st));
  }
  {
    GemmPlan p = plan_gemm(KC_DOWN, m, n_tok, ctx->n_cus);
    GemmArgs a = gemm_base(p, s, KC_DOWN, n_tok, m);
    a.W = l->wd;
    a.w_gstride = (long long)H * I;
    a.w_scale = l->wd_scale;
    a.ws_gstride = H;
    a.K = I;
    a.N = H;
    a.group_off = r.offsets;
    a.out = y;
    a.out_ld = H;
    if (fp8) {
      a.X = s.z8;
      a.x_ld = I;
      a.x_scale = s.z8_scale;
    } else {
      a.X = s.z;
      a.x_ld = I;
    }
    HookScope hs(th, KC_DOWN, st);
    SPA_HIP(launch_gemm(m->expert_dtype, XM_RAW, EPI_STORE, a, st));
  }
  return SPA_OK;
}

static spa_status op_combine(const spa_model_desc* m, const float* h, const float* y, const spa_route_bufs& r,
                             int n_tok, float* x_out, float* ss_out, int ss_ld, int k, hipStream_t st,
                             TimingHook* th) {
  CombineArgs a;
  a.h = h;
  a.y = y;
  a.w = r.topk_w;
  a.inv = r.inv;
  a.k = k;
  a.n_tok = n_tok;
  a.H = m->hidden;
  a.x_out = x_out;
  a.ss_out = ss_out;
  a.ss_ld = ss_ld;
  HookScope hs(th, KC_COMBINE, st);
  SPA_HIP(launch_combine(a, st));
  return SPA_OK;
}

// ---------------------------------------------------------------------------
// segments
// ---------------------------------------------------------------------------
spa_status run_segment_a(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int layer_index,
                         const spa_batch* b, int tok0, int n_tok, const WsLayout& W, const Slot& s, bool with_router,
                         bool first_layer, hipStream_t st, TimingHook* th) {
  spa_status rc;
  float* x = b->x + (size_t)tok0 * m->hidden;
  if (first_layer) {
    spa_route_bufs none{};
    rc = op_combine(m, x, nullptr, none, n_tok, x, s.ss_x, n_tok, 0, st, nullptr);
    if (rc) return rc;
  }
  if ((rc = op_qkv(ctx, m, l, b, tok0, n_tok, s.ss_x, n_tok, s.q, s, st, th))) return rc;
  if ((rc = op_attn(ctx, m, l, b, tok0, n_tok, s.q, s.o, W, s, st, th))) return rc;
  if ((rc = op_oproj(ctx, m, l, x, s.o, n_tok, s.h, s.ss_h, n_tok, s, st, th))) return rc;
  if (with_router) {
    int32_t* rec = b->topk_out ? b->topk_out + ((size_t)layer_index * b->batch + tok0) * m->top_k : nullptr;
    if ((rc = op_route(ctx, m, l, s.h, s.ss_h, n_tok, n_tok, s.logits, s.route, rec, s, st, th))) return rc;
  }
  return SPA_OK;
}

spa_status run_segment_b(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int layer_index,
                         const spa_batch* b, int tok0, int n_tok, const WsLayout& W, const Slot& s, bool with_router,
                         hipStream_t st, TimingHook* th) {
  (void)W;
  spa_status rc;
  float* x = b->x + (size_t)tok0 * m->hidden;
  if (!with_router) {
    int32_t* rec = b->topk_out ? b->topk_out + ((size_t)layer_index * b->batch + tok0) * m->top_k : nullptr;
    if ((rc = op_route(ctx, m, l, s.h, s.ss_h, n_tok, n_tok, s.logits, s.route, rec, s, st, th))) return rc;
  }
  if ((rc = op_expert(ctx, m, l, s.h, s.ss_h, n_tok, n_tok, s.route, s.y, s, st, th))) return rc;
  return op_combine(m, s.h, s.y, s.route, n_tok, x, s.ss_x, n_tok, m->top_k, st, th);
}

// ---------------------------------------------------------------------------
// argument checks
// ---------------------------------------------------------------------------
static spa_status check_batch(const spa_model_desc* m, const spa_batch* b) {
  if (!b) return fail(SPA_EINVAL, "batch is NULL");
  if (b->batch < 1) return fail(SPA_EINVAL, "batch must be >= 1");
  if (b->max_kv_len < 1) return fail(SPA_EINVAL, "max_kv_len must be >= 1");
  if (!b->kv_len || !b->kv_off || !b->kv_cap || !b->x) return fail(SPA_EINVAL, "batch pointer is NULL");
  if (((uintptr_t)b->x) & 15) return fail(SPA_EINVAL, "x must be 16-byte aligned");
  if (b->batch * m->top_k > 4096) return fail(SPA_EUNSUPPORTED, "batch * top_k above 4096 per call");
  return SPA_OK;
}

static spa_status check_layer(const spa_model_desc* m, const spa_layer* l) {
  if (!l) return fail(SPA_EINVAL, "layer is NULL");
  if (l->kind != SPA_FULL && l->kind != SPA_SLIDING) return fail(SPA_EINVAL, "bad layer kind");
  const void* ps[] = {l->wqkv, l->wo, l->wr, l->wgu, l->wd, l->gamma1, l->gamma2, l->sinks, l->k_cache, l->v_cache};
  for (const void* p : ps) {
    if (!p) return fail(SPA_EINVAL, "layer pointer is NULL");
    if (((uintptr_t)p) & 15) return fail(SPA_EINVAL, "layer tensors must be 16-byte aligned");
  }
  if (m->expert_dtype == SPA_E4M3 && (!l->wgu_scale || !l->wd_scale))
    return fail(SPA_EINVAL, "E4M3 experts need wgu_scale and wd_scale");
  return SPA_OK;
}

static spa_status check_ws(const spa_model_desc* m, int n_tok, int max_kv_len, int n_micro, void* ws,
                           size_t ws_bytes, WsLayout* out) {
  if (!ws) return fail(SPA_EINVAL, "workspace is NULL");
  if (((uintptr_t)ws) & 255) return fail(SPA_EINVAL, "workspace must be 256-byte aligned");
  WsLayout L = ws_layout(m, n_tok, max_kv_len, n_micro);
  if (ws_bytes < L.total)
    return fail(SPA_EWORKSPACE, "workspace too small: need " + std::to_string(L.total) + " bytes");
  *out = L;
  return SPA_OK;
}

}  // namespace spa

using namespace spa;

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* spa_last_error(void) { return g_err.c_str(); }

spa_status spa_init(int hip_device, spa_ctx** out) {
  if (!out) return fail(SPA_EINVAL, "out is NULL");
  int n = 0;
  SPA_HIP(hipGetDeviceCount(&n));
  if (hip_device < 0 || hip_device >= n) return fail(SPA_EINVAL, "no such HIP device");
  SPA_HIP(hipSetDevice(hip_device));
  spa_ctx* c = new spa_ctx();
  c->device = hip_device;
  hipError_t e = hipGetDeviceProperties(&c->prop, hip_device);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "hipGetDeviceProperties");
  }
  c->n_cus = c->prop.multiProcessorCount;
  if (strncmp(c->prop.gcnArchName, "gfx950", 6) != 0) {
    std::string arch = c->prop.gcnArchName;
    delete c;
    return fail(SPA_EUNSUPPORTED, "this library is built for gfx950, device is " + arch);
  }
  c->n_xcd = 8;
  *out = c;
  return SPA_OK;
}

spa_status spa_shutdown(spa_ctx* ctx) {
  delete ctx;
  return SPA_OK;
}

spa_status spa_device_cus(spa_ctx* ctx, int32_t* n) {
  if (!ctx || !n) return fail(SPA_EINVAL, "NULL argument");
  *n = ctx->n_cus;
  return SPA_OK;
}

spa_status spa_workspace_query(const spa_model_desc* m, int32_t batch, int32_t max_kv_len, int32_t n_micro,
                               size_t* bytes) {
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if (!bytes) return fail(SPA_EINVAL, "bytes is NULL");
  if (batch < 1 || n_micro < 1 || batch % n_micro) return fail(SPA_EINVAL, "n_micro must divide batch");
  if (max_kv_len < 1) return fail(SPA_EINVAL, "max_kv_len must be >= 1");
  *bytes = ws_layout(m, batch / n_micro, max_kv_len, n_micro).total;
  return SPA_OK;
}

spa_status spa_workspace_init(spa_ctx* ctx, const spa_model_desc* m, int32_t batch, int32_t max_kv_len,
                              int32_t n_micro, void* ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if (batch < 1 || n_micro < 1 || batch % n_micro) return fail(SPA_EINVAL, "n_micro must divide batch");
  WsLayout L;
  if ((rc = check_ws(m, batch / n_micro, max_kv_len, n_micro, ws, ws_bytes, &L))) return rc;
  return clear_counters(L, ws, (hipStream_t)stream);
}

spa_status spa_workspace_errors(spa_ctx* ctx, const void* ws, size_t ws_bytes, void* stream, int32_t* bits) {
  if (!ctx || !ws || !bits || ws_bytes < 4) return fail(SPA_EINVAL, "NULL argument");
  int v = 0;
  SPA_HIP(hipMemcpyAsync(&v, ws, 4, hipMemcpyDeviceToHost, (hipStream_t)stream));
  SPA_HIP(hipStreamSynchronize((hipStream_t)stream));
  *bits = v;
  return SPA_OK;
}

spa_status spa_kv_io(spa_ctx* ctx, const spa_model_desc* m, int32_t kind, void* k_cache, void* v_cache,
                     const spa_batch* b, const int32_t* seq, const int32_t* pos, int32_t n, void* k_rows,
                     void* v_rows, int32_t write, void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if (kind != SPA_FULL && kind != SPA_SLIDING) return fail(SPA_EINVAL, "bad kind");
  if (n < 0) return fail(SPA_EINVAL, "n < 0");
  if (n == 0) return SPA_OK;
  if (!k_cache || !v_cache || !seq || !pos || !k_rows || !v_rows) return fail(SPA_EINVAL, "NULL pointer");
  if (!b || b->batch < 1) return fail(SPA_EINVAL, "batch descriptor needed (sequence count)");
  if (kind == SPA_FULL && (!b->kv_off || !b->kv_cap)) return fail(SPA_EINVAL, "full layers need kv_off/kv_cap");
  KvIoArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_dtype = m->kv_dtype;
  a.kv_kind = kind == SPA_FULL ? KV_PACKED : KV_RING;
  a.kv_off = b ? (const long long*)b->kv_off : nullptr;
  a.kv_cap = b ? b->kv_cap : nullptr;
  a.window = m->window;
  a.n_kv_heads = m->n_kv_heads;
  a.head_dim = m->head_dim;
  a.seq = seq;
  a.pos = pos;
  a.n = n;
  a.n_seq = b->batch;
  a.k_rows = k_rows;
  a.v_rows = v_rows;
  a.write = write ? 1 : 0;
  SPA_HIP(launch_kv_io(a, (hipStream_t)stream));
  return SPA_OK;
}

spa_status spa_row_sumsq(spa_ctx* ctx, const spa_model_desc* m, const float* x, int32_t n_tok, float* ss,
                         void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if (!x || !ss || n_tok < 1) return fail(SPA_EINVAL, "bad argument");
  CombineArgs a;
  memset(&a, 0, sizeof(a));
  a.h = x;
  a.k = 0;
  a.n_tok = n_tok;
  a.H = m->hidden;
  a.x_out = const_cast<float*>(x);   // k == 0: rewrites each element with itself
  a.ss_out = ss;
  a.ss_ld = n_tok;
  SPA_HIP(launch_combine(a, (hipStream_t)stream));
  return SPA_OK;
}

#define SPA_OP_PROLOGUE(n_tok_expr)                                                      \
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");                                      \
  spa_status rc = validate_model(m);                                                     \
  if (rc) return rc;                                                                     \
  WsLayout W;                                                                            \
  if ((rc = check_ws(m, (n_tok_expr), max_kv, 1, ws, ws_bytes, &W))) return rc;          \
  Slot s = slot_ptrs(W, ws, 0);                                                          \
  hipStream_t st = (hipStream_t)stream;                                                  \
  if ((rc = clear_counters(W, ws, st))) return rc;

spa_status spa_qkv_append(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int32_t tok0,
                          int32_t n_tok, const float* ss_x, void* q_out, void* ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_batch(m, b);
  if (rc0) return rc0;
  if ((rc0 = check_layer(m, l))) return rc0;
  if (tok0 < 0 || n_tok < 1 || tok0 + n_tok > b->batch) return fail(SPA_EINVAL, "token range outside the batch");
  if (!ss_x || !q_out) return fail(SPA_EINVAL, "NULL pointer");
  const int max_kv = b->max_kv_len;
  SPA_OP_PROLOGUE(n_tok)
  return op_qkv(ctx, m, l, b, tok0, n_tok, ss_x, n_tok, q_out, s, st, nullptr);
}

spa_status spa_decode_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int32_t tok0,
                           int32_t n_tok, const void* q, void* o_out, void* ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_batch(m, b);
  if (rc0) return rc0;
  if ((rc0 = check_layer(m, l))) return rc0;
  if (tok0 < 0 || n_tok < 1 || tok0 + n_tok > b->batch) return fail(SPA_EINVAL, "token range outside the batch");
  if (!q || !o_out || (((uintptr_t)q) & 15)) return fail(SPA_EINVAL, "q / o_out NULL or misaligned");
  const int max_kv = b->max_kv_len;
  SPA_OP_PROLOGUE(n_tok)
  return op_attn(ctx, m, l, b, tok0, n_tok, q, o_out, W, s, st, nullptr);
}

spa_status spa_out_proj(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* x, const void* o,
                        int32_t n_tok, float* h_out, float* ss_h, void* ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_layer(m, l);
  if (rc0) return rc0;
  if (!x || !o || !h_out || !ss_h || n_tok < 1) return fail(SPA_EINVAL, "bad argument");
  if ((((uintptr_t)x) | ((uintptr_t)o) | ((uintptr_t)h_out)) & 15) return fail(SPA_EINVAL, "misaligned tensor");
  const int max_kv = 1;
  SPA_OP_PROLOGUE(n_tok)
  return op_oproj(ctx, m, l, x, o, n_tok, h_out, ss_h, n_tok, s, st, nullptr);
}

spa_status spa_moe_route(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* h, const float* ss_h,
                         int32_t n_tok, float* logits_out, const spa_route_bufs* r, int32_t* topk_rec, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_layer(m, l);
  if (rc0) return rc0;
  if (!h || !ss_h || !logits_out || !r || n_tok < 1) return fail(SPA_EINVAL, "bad argument");
  if (!r->topk_idx || !r->topk_w || !r->offsets || !r->row_tok || !r->row_slot || !r->inv)
    return fail(SPA_EINVAL, "route buffer is NULL");
  if (n_tok * m->top_k > 4096) return fail(SPA_EUNSUPPORTED, "n_tok * top_k above 4096");
  const int max_kv = 1;
  SPA_OP_PROLOGUE(n_tok)
  return op_route(ctx, m, l, h, ss_h, n_tok, n_tok, logits_out, *r, topk_rec, s, st, nullptr);
}

spa_status spa_moe_expert(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* h, const float* ss_h,
                          int32_t n_tok, const spa_route_bufs* r, float* y_out, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_layer(m, l);
  if (rc0) return rc0;
  if (!h || !ss_h || !r || !y_out || n_tok < 1) return fail(SPA_EINVAL, "bad argument");
  const int max_kv = 1;
  SPA_OP_PROLOGUE(n_tok)
  return op_expert(ctx, m, l, h, ss_h, n_tok, n_tok, *r, y_out, s, st, nullptr);
}

spa_status spa_moe_combine(spa_ctx* ctx, const spa_model_desc* m, const float* h, const float* y,
                           const spa_route_bufs* r, int32_t n_tok, float* x_out, float* ss_out, void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if (!h || !y || !r || !x_out || !ss_out || n_tok < 1) return fail(SPA_EINVAL, "bad argument");
  return op_combine(m, h, y, *r, n_tok, x_out, ss_out, n_tok, m->top_k, (hipStream_t)stream, nullptr);
}

spa_status spa_layer_forward(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int32_t layer_index,
                             const spa_batch* b, int32_t tok0, int32_t n_tok, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_batch(m, b);
  if (rc0) return rc0;
  if ((rc0 = check_layer(m, l))) return rc0;
  if (tok0 < 0 || n_tok < 1 || tok0 + n_tok > b->batch) return fail(SPA_EINVAL, "token range outside the batch");
  if (layer_index < 0 || layer_index >= m->n_layers) return fail(SPA_EINVAL, "layer_index out of range");
  const int max_kv = b->max_kv_len;
  SPA_OP_PROLOGUE(n_tok)
  if ((rc = run_segment_a(ctx, m, l, layer_index, b, tok0, n_tok, W, s, false, true, st, nullptr))) return rc;
  return run_segment_b(ctx, m, l, layer_index, b, tok0, n_tok, W, s, false, st, nullptr);
}

spa_status spa_temporal_run(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* layers, const spa_batch* b,
                            int32_t n_micro, void* ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if ((rc = check_batch(m, b))) return rc;
  if (!layers) return fail(SPA_EINVAL, "layers is NULL");
  for (int i = 0; i < m->n_layers; ++i)
    if ((rc = check_layer(m, &layers[i]))) return rc;
  if (n_micro < 1 || b->batch % n_micro) return fail(SPA_EINVAL, "n_micro must divide the batch");
  const int bm = b->batch / n_micro;
  WsLayout W;
  if ((rc = check_ws(m, bm, b->max_kv_len, n_micro, ws, ws_bytes, &W))) return rc;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = clear_counters(W, ws, st))) return rc;
  // the pipeline's dispatch order (layer, then microbatch), serialised on one stream
  for (int li = 0; li < m->n_layers; ++li) {
    for (int mu = 0; mu < n_micro; ++mu) {
      Slot s = slot_ptrs(W, ws, mu);
      if ((rc = run_segment_a(ctx, m, &layers[li], li, b, mu * bm, bm, W, s, false, li == 0, st, nullptr))) return rc;
      if ((rc = run_segment_b(ctx, m, &layers[li], li, b, mu * bm, bm, W, s, false, st, nullptr))) return rc;
    }
  }
  return SPA_OK;
}

}  // extern "C"
