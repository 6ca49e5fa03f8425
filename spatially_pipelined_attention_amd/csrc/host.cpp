// Host side of the C ABI: validation, workspace carving, operator launches,
// the layer's two segments, single-layer and temporal execution.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <unordered_map>

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
  if (m->n_resident > 128) return fail(SPA_EUNSUPPORTED, "more than 128 resident experts");
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
  if (m->hidden > 4096) return fail(SPA_EUNSUPPORTED, "hidden above 4096 (row kernels hold 4 columns per thread)");
  if (!(m->comm_latency_us >= 0.f && m->comm_latency_us <= 1000.f))
    return fail(SPA_EINVAL, "comm_latency_us must be in [0, 1000]");
  if (!(m->comm_gbps >= 0.f && m->comm_gbps <= 100000.f)) return fail(SPA_EINVAL, "comm_gbps must be in [0, 100000]");
  if (!(m->rope_theta >= 0.f && m->rope_theta <= 3.0e38f)) return fail(SPA_EINVAL, "rope_theta must be finite and >= 0");
  return SPA_OK;
}

bool comm_enabled(const spa_model_desc* m) { return m->comm_gbps > 0.f; }

// Payload bytes of the three collectives of one layer for n_tok tokens: the
// attention all-reduce carries the output projection's rows, dispatch the
// expert input rows (and their E4M3 scales), combine the expert output rows.
static size_t comm_bytes_allreduce(const spa_model_desc* m, int n_tok) {
  return (size_t)n_tok * m->hidden * esz_of(m->dense_dtype);
}
static size_t comm_bytes_dispatch(const spa_model_desc* m, int n_tok) {
  const size_t R = (size_t)n_tok * m->top_k;
  return R * m->hidden * esz_of(m->expert_dtype) + (m->expert_dtype == SPA_E4M3 ? R * 4 : 0);
}
static size_t comm_bytes_combine(const spa_model_desc* m, int n_tok) {
  return (size_t)n_tok * m->top_k * m->hidden * esz_of(m->dense_dtype);
}

spa_status launch_comm(spa_ctx* ctx, const void* src, void* dst, size_t copy_bytes, size_t bytes, double latency_us,
                       double gbps, hipStream_t st) {
  const double us = latency_us + (gbps > 0.0 ? (double)bytes / (gbps * 1e3) : 0.0);
  if (!(us >= 0.0 && us < 1e5)) return fail(SPA_EINVAL, "modelled communication time must be below 100 ms");
  const unsigned long long ticks = (unsigned long long)std::llround(us * ctx->wall_khz / 1000.0);
  SPA_HIP(launch_virtual_comm(src, dst, (long long)(copy_bytes / 16), ticks, st));
  return SPA_OK;
}

// Full layers of up to kDealMaxTok tokens run as an even split of the
// launch's blocks into deal_ranges() ranges (k_attn_dealt): its partial slots
// and the per-window merge table.
static bool dealt_launch(const spa_layer* l, int n_tok) { return l->kind == SPA_FULL && n_tok <= kDealMaxTok; }
static int deal_ranges(int device_cus) { return kDealRangesPerCu * device_cus; }
static size_t deal_part_bytes(int ranges, int n_tok, int Hkv, int G, int D) {
  return ((size_t)ranges + (size_t)n_tok * Hkv) * G * (D + 2) * 4 + (size_t)n_tok * Hkv * 2 * 4;
}

int max_chunks_for(int max_kv_len, const spa_model_desc* m) {
  int l = std::max(max_kv_len, m->window);
  return (l + kAttnChunk - 1) / kAttnChunk;
}

// Launch shapes depend only on tensor shapes (never on the CU pool), so a
// microbatch computes the same bits in every schedule.
static int pick_blk_rows(int need) {
  for (int r : {16, 32, 48, 64, 80}) if (need <= r) return r;
  return 128;
}

// Shape of one projection: rows per block (one W read serves them all),
// output columns per tile, and the split-K factor that gives the chip enough
// workgroups. Grouped (expert) products size the row block for the expected
// rows per expert plus two standard deviations of uniform routing, so an
// expert's W is streamed once with high probability.
GemmPlan plan_gemm(int kc, const spa_model_desc* m, int n_tok, int n_cus) {
  GemmPlan p{};
  int K = 0, N = 0, groups = 0;
  p.epi = EPI_PARTIAL;
  p.tile_cols = 64;
  switch (kc) {
    case KC_QKV: K = m->hidden; p.ks = ks_of(m->dense_dtype); N = (m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim; break;
    case KC_OPROJ: K = m->n_q_heads * m->head_dim; p.ks = ks_of(m->dense_dtype); N = m->hidden; break;
    case KC_ROUTER: K = m->hidden; p.ks = 16; N = m->n_experts; p.tile_cols = 16; break;
    case KC_GATEUP: K = m->hidden; p.ks = ks_of(m->expert_dtype); N = 2 * m->inter; groups = m->n_resident;
      p.epi = EPI_SWIGLU;
      break;
    case KC_DOWN: K = m->inter; p.ks = ks_of(m->expert_dtype); N = m->hidden; groups = m->n_resident; break;
    default: break;
  }
  p.n_groups = std::max(groups, 1);
  p.n_tiles = (N + p.tile_cols - 1) / p.tile_cols;
  p.part_ld = p.n_tiles * p.tile_cols;
  int busy_blocks;   // row blocks expected to hold rows
  if (groups == 0) {
#ifndef SPA_ROUTER_ROWS
#define SPA_ROUTER_ROWS 32
#endif
    // The router's fp32 activation rows outweigh its 16-column weight tiles
    // (rows / 16 activation loads per weight load), so up to 128 tokens its
    // row blocks are capped: the 1.5 MB of weights are then read up to 4
    // times, and each workgroup loads a quarter of the activations (at 64
    // tokens the 36-layer iteration measured about 50 us faster).
    const int rows_cap = kc == KC_ROUTER && n_tok <= 128 ? SPA_ROUTER_ROWS : 128;
    p.blk_rows = pick_blk_rows(std::min(n_tok, rows_cap));
    p.rb_stride = (n_tok + p.blk_rows - 1) / p.blk_rows;
    p.part_rows = n_tok;
    busy_blocks = p.rb_stride;
  } else {
    const int R = n_tok * m->top_k;
    const double mean = (double)R / groups;
    p.blk_rows = pick_blk_rows(std::max(1, (int)std::ceil(mean + 2.0 * std::sqrt(mean))));
    const int rb_all = (R + p.blk_rows - 1) / p.blk_rows;   // every row in one group
    p.rb_stride = std::min(groups * rb_all, rb_all + groups);
    p.part_rows = R;
    // groups expected to hold rows, times the blocks such a group needs
    const int per_group = std::max(1, (int)std::ceil(mean / p.blk_rows));
    busy_blocks = std::min(p.rb_stride, std::max(1, std::min(groups, R)) * per_group);
  }
  const int nks = K / p.ks;
  const int s_max = std::min(16, std::max(1, nks / 8));   // two k-steps per wave; the finish kernels sum <= 16
#ifndef SPA_GEMM_TARGET_X4
#define SPA_GEMM_TARGET_X4 5
#endif
  const int target = std::max(256, (n_cus * SPA_GEMM_TARGET_X4) / 4);
  int S = (target + p.n_tiles * busy_blocks - 1) / (p.n_tiles * busy_blocks);
  // A workgroup streams its k range at about one CU's share of the
  // bandwidth, so a grid a little larger than the CU count leaves the CUs
  // holding two workgroups to finish alone, and a smaller one leaves CUs
  // idle. The (tile width, split) pair is the one of least modelled time,
  // in units of the weight stream at full fill:
  //   ceil(w / n_cus) * n_cus / w          the busiest CU's share (w workgroups)
  //   * (1 + 0.6 * block rows / tile cols)  activation loads per weight byte
  //   + 4 * splits * rows per group / (K * weight element size)
  //                                         the fp32 split partials, written and
  //                                         read once (about half of it served
  //                                         by the last-level cache)
  // Dense products use 64-column tiles; expert products also 96 (at most 80
  // rows in registers) and 48 (not SwiGLU, whose tiles pair gate and up
  // halves). SwiGLU takes no split. Ties keep the wider tile, then the
  // smaller split. The router keeps its 16-column fp32 tiles and the target.
  if (kc != KC_ROUTER) {
    const double rows_per_group = groups == 0 ? (double)n_tok : (double)n_tok * m->top_k / groups;
    const double wbytes_per_k = (double)K * esz_of(groups == 0 ? m->dense_dtype : m->expert_dtype);
    const int s_lim = p.epi == EPI_SWIGLU ? 1 : s_max;
    double best = 1e30;
    for (int tc : {96, 64, 48}) {
      if ((groups == 0 || m->expert_dtype == SPA_F32) && tc != 64) continue;
      if ((tc == 96 && p.blk_rows > 80) || (tc == 48 && p.epi == EPI_SWIGLU)) continue;
      const int tiles = (N + tc - 1) / tc;
      for (int c = 1; c <= s_lim; ++c) {
        const double w = (double)tiles * busy_blocks * c;
        const double fill = std::ceil(w / n_cus) * n_cus / w;
        const double cost = fill * (1.0 + 0.6 * p.blk_rows / tc) + 4.0 * c * rows_per_group / wbytes_per_k;
        if (cost < best - 1e-9) {
          best = cost;
          p.tile_cols = tc;
          p.n_tiles = tiles;
          p.part_ld = tiles * tc;
          S = c;
        }
      }
    }
  }
  S = std::min(S, s_max);
  // Full 128-row blocks (hundreds of rows per expert, or 256 and more dense
  // rows): the LDS-tiled kernel, 128 weight rows per workgroup, its split
  // chosen for about two workgroups per CU (at most 6; SwiGLU takes none).
  const int wdt = groups == 0 ? m->dense_dtype : m->expert_dtype;
#ifndef SPA_GEMM_BIG
#define SPA_GEMM_BIG 1
#endif
  if (SPA_GEMM_BIG && kc != KC_ROUTER && wdt != SPA_F32 && p.blk_rows == 128 && (groups > 0 || n_tok >= 256)) {
    p.tile_cols = 128;
    p.n_tiles = (N + 127) / 128;
    p.part_ld = p.n_tiles * 128;
    const int tb = p.n_tiles * busy_blocks;
    S = std::min({6, s_max, std::max(1, (2 * n_cus + tb - 1) / tb)});
  }
  if (p.epi == EPI_SWIGLU) S = 1;
  p.S = std::max(1, S);
  if (kc == KC_DOWN && p.S == 1) p.epi = EPI_STORE;
  return p;
}

// Columns of the partial buffer of an N-column product: any tile width the
// plans use (16, 48, 64, 96, 128; all divide 384) pads N to at most this.
static size_t part_ld_bound(int N) { return (size_t)(N + 383) / 384 * 384; }

// Partial space for any call of up to n_tok tokens: the largest split any
// plan may choose (16, and at most an eighth of the k-steps) times the rows
// and padded columns of the product.
static size_t gemm_part_floats(const spa_model_desc* m, int n_tok) {
  size_t mx = 0;
  for (int kc : {KC_QKV, KC_OPROJ, KC_ROUTER, KC_DOWN}) {
    const GemmPlan p = plan_gemm(kc, m, n_tok, 1);
    int K = kc == KC_QKV || kc == KC_ROUTER ? m->hidden : (kc == KC_OPROJ ? m->n_q_heads * m->head_dim : m->inter);
    const int N = kc == KC_QKV ? (m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim
                               : (kc == KC_ROUTER ? m->n_experts : m->hidden);
    const size_t s_max = (size_t)std::min(16, std::max(1, K / p.ks / 8));
    mx = std::max(mx, s_max * p.part_rows * std::max((size_t)p.part_ld, part_ld_bound(N)));
  }
  return mx;
}

WsLayout ws_layout(const spa_model_desc* m, int n_tok, int max_kv_len, int n_micro) {
  WsLayout L{};
  const int H = m->hidden, Hq = m->n_q_heads, Hkv = m->n_kv_heads, D = m->head_dim;
  const int G = Hq / Hkv, k = m->top_k, E = m->n_experts, Er = m->n_resident, I = m->inter;
  const int R = n_tok * k;
  const size_t kv_esz = esz_of(m->kv_dtype), dn_esz = esz_of(m->dense_dtype);
  const bool fp8 = m->expert_dtype == SPA_E4M3, ebf = m->expert_dtype == SPA_BF16;
  L.n_slots = n_micro;
  L.n_tok = n_tok;
  L.max_chunks = max_chunks_for(max_kv_len, m);
  SlotLayout& s = L.s;
  size_t o = 0;
  s.xn = o; o = align256(o + (size_t)n_tok * H * dn_esz);
  s.q = o; o = align256(o + (size_t)n_tok * Hq * D * kv_esz);
  s.o = o; o = align256(o + (size_t)n_tok * Hq * D * kv_esz);
  s.h = o; o = align256(o + (size_t)n_tok * H * 4);
  s.hn_f32 = o; o = align256(o + (size_t)n_tok * H * 4);
  s.hn_bf16 = o; o = align256(o + (ebf ? (size_t)n_tok * H * 2 : 0));
  s.hn8 = o; o = align256(o + (fp8 ? (size_t)n_tok * H : 0));
  s.hn8_scale = o; o = align256(o + (fp8 ? (size_t)n_tok * 4 : 0));
  s.logits = o; o = align256(o + (size_t)n_tok * E * 4);
  s.topk_idx = o; o = align256(o + (size_t)R * 4);
  s.topk_w = o; o = align256(o + (size_t)R * 4);
  s.offsets = o; o = align256(o + (size_t)(Er + 1) * 4);
  s.row_tok = o; o = align256(o + (size_t)R * 4);
  s.row_slot = o; o = align256(o + (size_t)R * 4);
  s.inv = o; o = align256(o + (size_t)R * 4);
  s.xe_perm = o; o = align256(o + (size_t)R * H * esz_of(m->expert_dtype));
  s.xe_perm_scale = o; o = align256(o + (fp8 ? (size_t)R * 4 : 0));
  s.z = o; o = align256(o + (size_t)R * I * (ebf ? 2 : 4));
  s.z8 = o; o = align256(o + (fp8 ? (size_t)R * I : 0));
  s.z8_scale = o; o = align256(o + (fp8 ? (size_t)R * 4 : 0));
  s.y = o; o = align256(o + (size_t)R * H * 4);
  s.attn_part = o; o = align256(o + std::max((size_t)n_tok * Hkv * L.max_chunks * G * (D + 2) * 4,
                                             deal_part_bytes(kDealMaxRanges, n_tok, Hkv, G, D)));
  s.gemm_part = o; o = align256(o + gemm_part_floats(m, n_tok) * 4);
  s.comm = o;
  if (comm_enabled(m))
    o = align256(o + std::max({comm_bytes_allreduce(m, n_tok), comm_bytes_dispatch(m, n_tok),
                               comm_bytes_combine(m, n_tok)}));
  s.bytes = o;
  L.err = 0;
  L.slot0 = kHeaderWords * 4;
  L.slot_bytes = s.bytes;
  L.total = L.slot0 + (size_t)n_micro * s.bytes;
  return L;
}

Slot slot_ptrs(const WsLayout& L, void* ws, int slot) {
  Slot s{};
  char* b = (char*)ws + L.slot0 + (size_t)slot * L.slot_bytes;
  const SlotLayout& o = L.s;
  s.base = b;
  s.err = (int*)((char*)ws + L.err);
  // two hand-off counters of the MoE-head launch per slot, and one arrival
  // counter of the routing launch, in the header words that every run clears
  // (words 32..63: slots 0..15; words 64..127: slots 0..63)
  s.head_ctr = slot < 16 ? (unsigned*)((char*)ws + L.err) + 32 + 2 * slot : nullptr;
  s.route_ctr = slot < 64 ? (unsigned*)((char*)ws + L.err) + 64 + slot : nullptr;
  s.xn = b + o.xn;
  s.q = b + o.q;
  s.o = b + o.o;
  s.h = (float*)(b + o.h);
  s.hn_f32 = (float*)(b + o.hn_f32);
  s.hn_bf16 = (uint16_t*)(b + o.hn_bf16);
  s.hn8 = (uint8_t*)(b + o.hn8);
  s.hn8_scale = (float*)(b + o.hn8_scale);
  s.logits = (float*)(b + o.logits);
  s.route.topk_idx = (int32_t*)(b + o.topk_idx);
  s.route.topk_w = (float*)(b + o.topk_w);
  s.route.offsets = (int32_t*)(b + o.offsets);
  s.route.row_tok = (int32_t*)(b + o.row_tok);
  s.route.row_slot = (int32_t*)(b + o.row_slot);
  s.route.inv = (int32_t*)(b + o.inv);
  s.z = b + o.z;
  s.z8 = (uint8_t*)(b + o.z8);
  s.z8_scale = (float*)(b + o.z8_scale);
  s.xe_perm = b + o.xe_perm;
  s.xe_perm_scale = (float*)(b + o.xe_perm_scale);
  s.y = (float*)(b + o.y);
  s.attn_part = (float*)(b + o.attn_part);
  s.gemm_part = (float*)(b + o.gemm_part);
  s.comm = b + o.comm;
  return s;
}

static std::mutex g_cus_mu;
static std::unordered_map<hipStream_t, int> g_stream_cus;

void register_stream_cus(hipStream_t st, int n_cus) {
  std::lock_guard<std::mutex> lk(g_cus_mu);
  g_stream_cus[st] = n_cus;
}

void unregister_stream_cus(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_cus_mu);
  g_stream_cus.erase(st);
}

int stream_cus(hipStream_t st, int fallback) {
  std::lock_guard<std::mutex> lk(g_cus_mu);
  const auto it = g_stream_cus.find(st);
  return it == g_stream_cus.end() ? fallback : it->second;
}

spa_status clear_errors(void* ws, hipStream_t st) {
  SPA_HIP(launch_fill_i32((int*)ws, kHeaderWords, 0, st));
  return SPA_OK;
}

// ---------------------------------------------------------------------------
// timing hook: events around every launch of the timed kernel class
// ---------------------------------------------------------------------------
// Timing events need no system-scope release: they only order against work
// on the same device, and the release would flush L2 between kernels.
#ifndef SPA_TIMING_EVENT_FLAGS
#define SPA_TIMING_EVENT_FLAGS hipEventDisableSystemFence
#endif

struct HookScope {
  TimingHook* th;
  hipStream_t st;
  bool on;
  bool ext;          // the launch itself records the pair (hipExtLaunchKernel timestamps)
  hipEvent_t e0 = nullptr, e1 = nullptr;
  unsigned long long* span_slot = nullptr;   // device-clock span of this launch
  HookScope(TimingHook* t, int cls, hipStream_t s, bool in_launch = false)
      : th(t), st(s), on(t && t->cls == cls && t->evs && t->pool), ext(in_launch) {
    if (!on) return;
    if (ext && th->span) {   // the kernel records its own span: no events
      on = false;
      if (*th->span_used < th->span_cap) span_slot = th->span + (size_t)kSpanWords * (*th->span_used)++;
      return;
    }
    e0 = take();
    e1 = take();
    th->evs->push_back(e0);
    th->evs->push_back(e1);
    if (!ext) (void)hipEventRecord(e0, st);
  }
  hipEvent_t start() const { return on && ext ? e0 : nullptr; }
  hipEvent_t stop() const { return on && ext ? e1 : nullptr; }
  hipEvent_t take() {
    if (th->pool->empty()) {
      hipEvent_t e;
      (void)hipEventCreateWithFlags(&e, SPA_TIMING_EVENT_FLAGS);
      return e;
    }
    hipEvent_t e = th->pool->back();
    th->pool->pop_back();
    return e;
  }
  ~HookScope() {
    if (on && !ext) (void)hipEventRecord(e1, st);
  }
};

// ---------------------------------------------------------------------------
// operators (explicit pointers; scratch from slot s)
// ---------------------------------------------------------------------------
static GemmArgs gemm_args(const GemmPlan& p, const Slot& s, int n_tok) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.n_tiles = p.n_tiles;
  a.tile_cols = p.tile_cols;
  a.blk_rows = p.blk_rows;
  a.n_groups = p.n_groups;
  a.S = p.S;
  a.rb_stride = p.rb_stride;
  a.n_rows = n_tok;
  a.part = s.gemm_part;
  a.part_rows = p.part_rows;
  a.part_ld = p.part_ld;
  return a;
}

static PartView view_of(const GemmPlan& p, const Slot& s) {
  PartView v;
  v.part = s.gemm_part;
  v.S = p.S;
  v.rows = p.part_rows;
  v.ld = p.part_ld;
  return v;
}

// Norm + QKV: q and the new K/V (cache append) from xn.
// kmajor: the activation input (xn / o) is k-step-major over the call's rows,
// as the pipeline's own slot buffers are; the single-operator entry points
// take and return row-major tensors.
// fold_finish: the product only; the sliding attention's one-wave-per-window
// kernel sums its partials and appends K/V itself (qkv_folds).
static spa_status op_qkv(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0,
                         int n_tok, const void* xn, void* q_out, const Slot& s, hipStream_t st, TimingHook* th,
                         bool kmajor = false, bool fold_finish = false) {
  const GemmPlan p = plan_gemm(KC_QKV, m, n_tok, ctx->n_cus);
  GemmArgs a = gemm_args(p, s, n_tok);
  a.W = l->wqkv;
  a.K = m->hidden;
  a.N = (m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim;
  a.X = xn;
  a.x_rstride = kmajor ? 64 : (long long)m->hidden * esz_of(m->dense_dtype);
  a.x_kstride = kmajor ? (long long)n_tok * 64 : 64;
  QkvFinishArgs f;
  memset(&f, 0, sizeof(f));
  f.pv = view_of(p, s);
  f.n_tok = n_tok;
  f.n_q_heads = m->n_q_heads;
  f.n_kv_heads = m->n_kv_heads;
  f.head_dim = m->head_dim;
  f.q_out = q_out;
  f.kv_dtype = m->kv_dtype;
  f.kv_kind = l->kind == SPA_FULL ? KV_PACKED : KV_RING;
  f.k_cache = l->k_cache;
  f.v_cache = l->v_cache;
  f.kv_len = b->kv_len;
  f.kv_off = (const long long*)b->kv_off;
  f.kv_cap = b->kv_cap;
  f.window = m->window;
  f.tok0 = tok0;
  f.err = s.err;
  f.rope_theta = m->rope_theta;
  HookScope hs(th, KC_QKV, st);
  SPA_HIP(launch_gemm(m->dense_dtype, EPI_PARTIAL, a, st));
  if (!fold_finish) SPA_HIP(launch_qkv_finish(f, st));
  return SPA_OK;
}

// Chunk cap for attention: the largest of 4096 .. 512 that still gives at
// least two workgroups per CU at the batch's longest sequence (long chunks
// stream longer and leave fewer partials to merge; a window is then cut into
// equal chunks below the cap). Depends only on shapes and the device, never
// on the CU pool, so every schedule computes the same partials.
#ifndef SPA_ATTN_WGS_PER_CU
#define SPA_ATTN_WGS_PER_CU 2
#endif
static int attn_chunk(const spa_model_desc* m, const spa_batch* b, int n_tok, int n_cus) {
  for (int c = 4096; c > kAttnChunk; c >>= 1) {
    const long long wgs = (long long)n_tok * m->n_kv_heads * ((b->max_kv_len + c - 1) / c);
    if (wgs >= (long long)SPA_ATTN_WGS_PER_CU * n_cus) return c;
  }
  return kAttnChunk;
}

static AttnArgs attn_args(const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0, int n_tok,
                          const void* q, void* o, const WsLayout& W, const Slot& s, int n_cus) {
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
  a.chunk = l->kind == SPA_FULL ? attn_chunk(m, b, n_tok, n_cus) : kAttnChunk;
  // the workspace holds max_chunks_for() partials at the smallest chunk
  a.max_chunks = l->kind == SPA_FULL ? std::min(W.max_chunks, (b->max_kv_len + a.chunk - 1) / a.chunk)
                                     : (m->window + kAttnChunk - 1) / kAttnChunk;
  a.part = s.attn_part;
  a.o = o;
  a.err = s.err;
  a.stream_kv = 1;
  return a;
}

#ifndef SPA_ATTN_WAVE_PER_4CU
#define SPA_ATTN_WAVE_PER_4CU 2
#endif
// Sliding layers with at least SPA_ATTN_WAVE_PER_4CU windows per 4 CUs of the
// device (so the choice, and the results, never depend on the pool): one wave
// per window (k_attn_wave).
static bool sliding_wave(const spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int n_tok) {
  return l->kind == SPA_SLIDING && m->window <= 256 && SPA_ATTN_WAVE_PER_4CU >= 0 &&
         4LL * n_tok * m->n_kv_heads >= (long long)SPA_ATTN_WAVE_PER_4CU * ctx->n_cus;
}

#ifndef SPA_ATTN_FOLD_QKV
#define SPA_ATTN_FOLD_QKV 1
#endif
// Layers whose QKV finish runs inside the one-wave-per-window attention
// kernel (bf16 KV, no RoPE, 8 query heads per KV head, at most kFoldMaxSplits
// QKV splits): the finish kernel's launch is saved, and the attention
// computes exactly what it would have read. (Full layers keep the finish
// kernel: folded into the even split, every piece re-sums its q and the
// kernel's registers grow, and the iteration was slower.)
static bool qkv_folds(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int n_tok) {
  return SPA_ATTN_FOLD_QKV && sliding_wave(ctx, m, l, n_tok) && m->kv_dtype == SPA_BF16 && !(m->rope_theta > 0.f) &&
         m->head_dim == 64 && m->n_q_heads == 8 * m->n_kv_heads &&
         plan_gemm(KC_QKV, m, n_tok, ctx->n_cus).S <= kFoldMaxSplits;
}

// qkv: the QKV split partials when the finish is folded into the attention
// (qkv_folds), else null.
static spa_status op_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0, int n_tok,
                          const void* q, void* o, const WsLayout& W, const Slot& s, hipStream_t st, TimingHook* th,
                          bool kmajor = false, const PartView* qkv = nullptr) {
  AttnArgs a = attn_args(m, l, b, tok0, n_tok, q, o, W, s, ctx->n_cus);
  a.o_kmajor_rows = kmajor ? n_tok : 0;
  // full layers: the launch's blocks cut into ranges fixed by the device,
  // taken by two resident workgroups per CU of the stream's pool (the ranges,
  // and so the results, are the same for every pool)
  if (sliding_wave(ctx, m, l, n_tok)) a.wave_windows = 1;
  if (qkv) {
    if (!a.wave_windows) return fail(SPA_EINVAL, "the QKV finish folds only into one-wave-per-window attention");
    a.qkv = *qkv;
  }
  if (dealt_launch(l, n_tok)) {
    const int G = m->n_q_heads / m->n_kv_heads;
    a.deal_wgs = kDealWgsPerCu * stream_cus(st, ctx->n_cus);
    a.deal_v = deal_ranges(ctx->n_cus);
    if (a.deal_v > kDealMaxRanges) return fail(SPA_EUNSUPPORTED, "device has more CUs than the attention split supports");
    a.deal_tab = (int*)(a.part + ((size_t)a.deal_v + (size_t)n_tok * m->n_kv_heads) * G * (m->head_dim + 2));
  }
  {
    // the attention kernel alone, timed by its own dispatch (start/stop events of the launch)
    HookScope hs(th, l->kind == SPA_FULL ? KC_ATTN_FULL : KC_ATTN_SLIDING, st, true);
    a.tspan = hs.span_slot;
    SPA_HIP(launch_attn(a, st, hs.start(), hs.stop()));
  }
  if (a.deal_v > 0 || a.max_chunks > 1) SPA_HIP(launch_attn_merge(a, st));
  return SPA_OK;
}

static spa_status op_comm(spa_ctx* ctx, const spa_model_desc* m, const void* src, size_t copy_bytes, size_t bytes,
                          const Slot& s, hipStream_t st, TimingHook* th);

// Output proj + Add + Norm: h = x + o Wo^T, hn = RMSNorm(h) gamma2 (fp32, and
// the expert input format when hn_bf16 / hn8 are given). The split product's
// and the finish kernel's arguments.
static void oproj_args(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* x, const void* o,
                       int n_tok, float* h, float* hn, uint16_t* hn_bf16, uint8_t* hn8, float* hn8_scale,
                       const Slot& s, bool kmajor, GemmArgs* ga, OprojFinishArgs* fa) {
  const GemmPlan p = plan_gemm(KC_OPROJ, m, n_tok, ctx->n_cus);
  GemmArgs a = gemm_args(p, s, n_tok);
  a.W = l->wo;
  a.K = m->n_q_heads * m->head_dim;
  a.N = m->hidden;
  a.X = o;
  a.x_rstride = kmajor ? 64 : (long long)m->n_q_heads * m->head_dim * esz_of(m->dense_dtype);
  a.x_kstride = kmajor ? (long long)n_tok * 64 : 64;
  OprojFinishArgs f;
  memset(&f, 0, sizeof(f));
  f.pv = view_of(p, s);
  f.n_tok = n_tok;
  f.H = m->hidden;
  f.x = x;
  f.h_out = h;
  f.gamma = l->gamma2;
  f.eps = m->eps;
  f.hn_f32 = hn;
  f.hn_bf16 = hn_bf16;
  f.hn_e4m3 = hn8;
  f.hn_scale = hn8_scale;
  *ga = a;
  *fa = f;
}

static spa_status op_oproj(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* x, const void* o,
                           int n_tok, float* h, float* hn, uint16_t* hn_bf16, uint8_t* hn8, float* hn8_scale,
                           const Slot& s, hipStream_t st, TimingHook* th, bool kmajor = false) {
  GemmArgs a;
  OprojFinishArgs f;
  oproj_args(ctx, m, l, x, o, n_tok, h, hn, hn_bf16, hn8, hn8_scale, s, kmajor, &a, &f);
  HookScope hs(th, KC_OPROJ, st);
  SPA_HIP(launch_gemm(m->dense_dtype, EPI_PARTIAL, a, st));
  SPA_HIP(launch_oproj_finish(f, st));
  return SPA_OK;
}

// The expert input rows (bf16 / E4M3 / fp32, by expert dtype) of a slot.
static const void* expert_input(const spa_model_desc* m, const Slot& s) {
  return m->expert_dtype == SPA_BF16 ? (const void*)s.hn_bf16
         : m->expert_dtype == SPA_E4M3 ? (const void*)s.hn8
                                       : (const void*)s.hn_f32;
}

// Router GEMV, top-k and the dispatch permutation. gather: also gather the
// slot's expert input rows into dispatch order (s.xe_perm) in the same
// kernel. The router product's and the routing kernels' arguments.
// Whether the routing gathers the expert input rows into dispatch order: the
// virtual dispatch endpoint sends the gathered rows; otherwise the gate/up
// product reads them in place through the row map (measured faster than the
// gather: the permutation kernel then moves no rows, and the product's
// row-major activation fragments cost it about 0.5 us).
static bool route_gathers(const spa_model_desc* m) { return comm_enabled(m); }

static void route_args(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* hn, int n_tok,
                       float* logits, const spa_route_bufs& r, int32_t* topk_rec, const Slot& s, bool gather,
                       GemmArgs* ga, RouteArgs* ra_out, GemmPlan* plan) {
  const GemmPlan p = plan_gemm(KC_ROUTER, m, n_tok, ctx->n_cus);
  GemmArgs a = gemm_args(p, s, n_tok);
  a.W = l->wr;
  a.K = m->hidden;
  a.N = m->n_experts;
  a.X = hn;
  a.x_rstride = (long long)m->hidden * 4;
  a.x_kstride = 64;
  RouteArgs ra;
  memset(&ra, 0, sizeof(ra));
  ra.pv = view_of(p, s);
  ra.n_tok = n_tok;
  ra.E = m->n_experts;
  ra.k = m->top_k;
  ra.E_res = m->n_resident;
  ra.logits = logits;
  ra.topk_idx = r.topk_idx;
  ra.topk_w = r.topk_w;
  ra.topk_rec = topk_rec;
  ra.offsets = r.offsets;
  ra.row_tok = r.row_tok;
  ra.row_slot = r.row_slot;
  ra.inv = r.inv;
#ifndef SPA_ROUTE_ONE_LAUNCH
#define SPA_ROUTE_ONE_LAUNCH 1
#endif
  ra.arrive = SPA_ROUTE_ONE_LAUNCH && !gather ? s.route_ctr : nullptr;
  if (gather) {
    const bool fp8 = m->expert_dtype == SPA_E4M3;
    ra.gsrc = expert_input(m, s);
    ra.gK = m->hidden;
    ra.gesz = esz_of(m->expert_dtype);
    ra.gdst = s.xe_perm;
    ra.gsrc_scale = fp8 ? s.hn8_scale : nullptr;
    ra.gdst_scale = fp8 ? s.xe_perm_scale : nullptr;
  }
  *ga = a;
  *ra_out = ra;
  if (plan) *plan = p;
}

static spa_status op_route(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* hn, int n_tok,
                           float* logits, const spa_route_bufs& r, int32_t* topk_rec, const Slot& s, hipStream_t st,
                           TimingHook* th, bool gather = false) {
  GemmArgs a;
  RouteArgs ra;
  route_args(ctx, m, l, hn, n_tok, logits, r, topk_rec, s, gather, &a, &ra, nullptr);
  HookScope hs(th, KC_ROUTER, st);
  SPA_HIP(launch_gemm(DT_F32, EPI_PARTIAL, a, st));
  SPA_HIP(launch_route(ra, st));
  return SPA_OK;
}

// Output projection through the gather of the expert rows, with the MoE head
// (finish, router, top-k, permutation and gather) as one persistent launch
// after the output projection's split product: the same bits as the
// separate launches. Those run instead when the head does not apply: no
// counter slot, split counts or router rows outside its instances, the
// virtual communication endpoints on (the all-reduce sits between the
// projection and the router), or fuse false.
static spa_status op_oproj_route(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* x, int n_tok,
                                 const Slot& s, int32_t* rec, bool fuse, hipStream_t st, TimingHook* th) {
  const bool fp8 = m->expert_dtype == SPA_E4M3, ebf = m->expert_dtype == SPA_BF16;
  MoeHeadArgs h;
  memset(&h, 0, sizeof(h));
  GemmArgs oa;
  GemmPlan rp;
  oproj_args(ctx, m, l, x, s.o, n_tok, s.h, s.hn_f32, ebf ? s.hn_bf16 : nullptr, fp8 ? s.hn8 : nullptr,
             fp8 ? s.hn8_scale : nullptr, s, true, &oa, &h.of);
  route_args(ctx, m, l, s.hn_f32, n_tok, s.logits, s.route, rec, s, true, &h.router, &h.ra, &rp);   // the head gathers
  const bool use = fuse && s.head_ctr && !comm_enabled(m) && moe_head_supported(h.of.pv.S, h.ra.pv.S, rp.blk_rows);
  if (!use) {
    spa_status rc = op_oproj(ctx, m, l, x, s.o, n_tok, s.h, s.hn_f32, ebf ? s.hn_bf16 : nullptr, fp8 ? s.hn8 : nullptr,
                             fp8 ? s.hn8_scale : nullptr, s, st, th, true);
    if (rc) return rc;
    const size_t ar = comm_bytes_allreduce(m, n_tok);
    if ((rc = op_comm(ctx, m, s.h, ar, ar, s, st, th))) return rc;   // attention all-reduce
    return op_route(ctx, m, l, s.hn_f32, n_tok, s.logits, s.route, rec, s, st, th, route_gathers(m));
  }
  h.n_router_tiles = rp.n_tiles * rp.rb_stride * rp.S;
  h.ctr = s.head_ctr;
  h.err = s.err;
  // at most one workgroup per CU of the stream's pool, so every workgroup is
  // resident while the others wait at a hand-off
  const int G = std::max(1, std::min(64, stream_cus(st, ctx->n_cus)));
  {
    HookScope hs(th, KC_OPROJ, st);
    SPA_HIP(launch_gemm(m->dense_dtype, EPI_PARTIAL, oa, st));
  }
  HookScope hs(th, KC_ROUTER, st);
  SPA_HIP(launch_moe_head(h, G, st));
  return SPA_OK;
}

// Experts: gate/up + SwiGLU, then down. xe: the expert input rows per token
// (bf16 / fp32 / E4M3 with xe_scale). Leaves y plain (S = 1) or as partials.
// Where the gate/up product finds its expert input rows: gathered into
// dispatch order (k-step-major) by the routing, to be gathered here, or read
// in place from the per-token rows through the row map (row_tok).
enum class ExpertRows { kGather, kGathered, kInPlace };

static spa_status op_expert(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const void* xe,
                            const float* xe_scale, int n_tok, const spa_route_bufs& r, float* y_plain, const Slot& s,
                            hipStream_t st, TimingHook* th, GemmPlan* down_plan,
                            ExpertRows rows = ExpertRows::kGather) {
  const int H = m->hidden, I = m->inter, R = n_tok * m->top_k;
  const bool fp8 = m->expert_dtype == SPA_E4M3;
  {
    const GemmPlan p = plan_gemm(KC_GATEUP, m, n_tok, ctx->n_cus);
    GemmArgs a = gemm_args(p, s, n_tok);
    a.W = l->wgu;
    a.w_gstride = (long long)2 * I * H;
    a.w_scale = l->wgu_scale;
    a.ws_gstride = 2 * I;
    a.K = H;
    a.N = I;
    a.inter = I;
    a.group_off = r.offsets;
    if (rows == ExpertRows::kInPlace) {
      // the per-token rows, row-major, through the row map
      a.X = xe;
      a.row_src = r.row_tok;
      a.x_rstride = (long long)H * esz_of(m->expert_dtype);
      a.x_kstride = 64;
      a.x_scale = fp8 ? xe_scale : nullptr;
    } else {
      // expert rows gathered in dispatch order, k-step-major: one 16-row X
      // fragment of a k-step is 1 KB of contiguous memory
      a.X = s.xe_perm;
      a.x_rstride = 64;
      a.x_kstride = (long long)R * 64;
      a.x_scale = fp8 ? s.xe_perm_scale : nullptr;
    }
    a.out = s.z;
    a.out_ld = I;
    a.out_kmajor_rows = R;
    a.out_dtype = m->expert_dtype == SPA_BF16 ? DT_BF16 : DT_F32;
    HookScope hs(th, KC_GATEUP, st);
    if (rows == ExpertRows::kGather)
      SPA_HIP(launch_gather_kmajor(xe, r.row_tok, R, H, esz_of(m->expert_dtype), s.xe_perm, fp8 ? xe_scale : nullptr,
                                   fp8 ? s.xe_perm_scale : nullptr, st));
    SPA_HIP(launch_gemm(m->expert_dtype, EPI_SWIGLU, a, st));
  }
  {
    const GemmPlan p = plan_gemm(KC_DOWN, m, n_tok, ctx->n_cus);
    GemmArgs a = gemm_args(p, s, n_tok);
    a.W = l->wd;
    a.w_gstride = (long long)H * I;
    a.w_scale = l->wd_scale;
    a.ws_gstride = H;
    a.K = I;
    a.N = H;
    a.group_off = r.offsets;
    a.out = y_plain;
    a.out_ld = H;
    HookScope hs(th, KC_DOWN, st);
    if (fp8) {
      CvtArgs c;
      memset(&c, 0, sizeof(c));
      c.x = (const float*)s.z;
      c.n_rows = R;
      c.n_cols = I;
      c.dtype = DT_E4M3;
      c.out = s.z8;
      c.scales = s.z8_scale;
      c.kmajor_rows = R;
      c.n_cus = ctx->n_cus;
      SPA_HIP(launch_cvt_rows(c, st));
      a.X = s.z8;
      a.x_scale = s.z8_scale;
    } else {
      a.X = s.z;
    }
    a.x_rstride = 64;                       // z is k-step-major over the R dispatch rows
    a.x_kstride = (long long)R * 64;
    SPA_HIP(launch_gemm(m->expert_dtype, p.epi, a, st));
    if (down_plan) *down_plan = p;
  }
  return SPA_OK;
}

static CombineArgs combine_args(const spa_model_desc* m, const float* h, const float* y, const GemmPlan* ypart,
                                const Slot* s, const spa_route_bufs& r, int n_tok, float* x_out,
                                const float* gamma_next, void* xn_out) {
  CombineArgs a;
  memset(&a, 0, sizeof(a));
  a.h = h;
  a.y = y;
  if (!y && ypart && s) {
    a.ypv = view_of(*ypart, *s);
    a.y_group_off = r.offsets;
    a.y_n_groups = m->n_resident;
  }
  a.w = r.topk_w;
  a.inv = r.inv;
  a.k = (y || ypart) ? m->top_k : 0;
  a.n_tok = n_tok;
  a.H = m->hidden;
  a.x_out = x_out;
  a.gamma_next = gamma_next;
  a.eps = m->eps;
  a.xn_out = xn_out;
  a.xn_dtype = m->dense_dtype;
  return a;
}

static spa_status op_combine(const spa_model_desc* m, const float* h, const float* y, const GemmPlan* ypart,
                             const Slot* s, const spa_route_bufs& r, int n_tok, float* x_out, const float* gamma_next,
                             void* xn_out, hipStream_t st, TimingHook* th, bool kmajor = false) {
  CombineArgs a = combine_args(m, h, y, ypart, s, r, n_tok, x_out, gamma_next, xn_out);
  a.xn_kmajor_rows = kmajor ? n_tok : 0;
  HookScope hs(th, KC_COMBINE, st);
  SPA_HIP(launch_combine(a, st));
  return SPA_OK;
}

// The virtual endpoint of one collective of the layer (nothing when the
// model has no communication): copies the payload's 16-byte words from src
// (a slot buffer at least that long) and lasts the payload's modelled time.
static spa_status op_comm(spa_ctx* ctx, const spa_model_desc* m, const void* src, size_t copy_bytes, size_t bytes,
                          const Slot& s, hipStream_t st, TimingHook* th) {
  if (!comm_enabled(m)) return SPA_OK;
  HookScope hs(th, KC_COMM, st);
  return launch_comm(ctx, src, s.comm, copy_bytes & ~(size_t)15, bytes, m->comm_latency_us, m->comm_gbps, st);
}

// ---------------------------------------------------------------------------
// segments of one layer on one microbatch slot
// ---------------------------------------------------------------------------
spa_status run_segment_a(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int layer_index,
                         const spa_layer* next, const spa_batch* b, int tok0, int n_tok, const WsLayout& W,
                         const Slot& s, bool with_router, bool first_layer, hipStream_t st, TimingHook* th,
                         bool fuse_head) {
  (void)next;
  spa_status rc;
  float* x = b->x + (size_t)tok0 * m->hidden;
  if (first_layer) {   // RMSNorm of the incoming residual rows
    spa_route_bufs none{};
    if ((rc = op_combine(m, x, nullptr, nullptr, nullptr, none, n_tok, x, l->gamma1, s.xn, st, nullptr, true))) return rc;
  }
  const bool fold = qkv_folds(ctx, m, l, n_tok);
  const PartView qkv_parts = view_of(plan_gemm(KC_QKV, m, n_tok, ctx->n_cus), s);
  if ((rc = op_qkv(ctx, m, l, b, tok0, n_tok, s.xn, s.q, s, st, th, true, fold))) return rc;
  if ((rc = op_attn(ctx, m, l, b, tok0, n_tok, s.q, s.o, W, s, st, th, true, fold ? &qkv_parts : nullptr))) return rc;
  if (with_router) {
    int32_t* rec = b->topk_out ? b->topk_out + ((size_t)layer_index * b->batch + tok0) * m->top_k : nullptr;
    return op_oproj_route(ctx, m, l, x, n_tok, s, rec, fuse_head, st, th);
  }
  const bool fp8 = m->expert_dtype == SPA_E4M3, ebf = m->expert_dtype == SPA_BF16;
  if ((rc = op_oproj(ctx, m, l, x, s.o, n_tok, s.h, s.hn_f32, ebf ? s.hn_bf16 : nullptr, fp8 ? s.hn8 : nullptr,
                     fp8 ? s.hn8_scale : nullptr, s, st, th, true)))
    return rc;
  const size_t ar = comm_bytes_allreduce(m, n_tok);
  return op_comm(ctx, m, s.h, ar, ar, s, st, th);   // attention all-reduce
}

// The layer in three pieces around its attention (the Macro cut):
// before = [first layer: RMSNorm of x] + QKV and KV append; attention;
// after = output projection, router, experts, combine.
spa_status run_layer_before_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b,
                                 int tok0, int n_tok, const Slot& s, bool first_layer, hipStream_t st,
                                 TimingHook* th) {
  spa_status rc;
  float* x = b->x + (size_t)tok0 * m->hidden;
  if (first_layer) {
    spa_route_bufs none{};
    if ((rc = op_combine(m, x, nullptr, nullptr, nullptr, none, n_tok, x, l->gamma1, s.xn, st, nullptr, true))) return rc;
  }
  return op_qkv(ctx, m, l, b, tok0, n_tok, s.xn, s.q, s, st, th, true, qkv_folds(ctx, m, l, n_tok));
}

// (with the QKV finish folded in, the attention reads the QKV partials, which
// the slot keeps until its output projection)
spa_status run_layer_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0,
                          int n_tok, const WsLayout& W, const Slot& s, hipStream_t st, TimingHook* th) {
  const PartView qkv_parts = view_of(plan_gemm(KC_QKV, m, n_tok, ctx->n_cus), s);
  return op_attn(ctx, m, l, b, tok0, n_tok, s.q, s.o, W, s, st, th, true,
                 qkv_folds(ctx, m, l, n_tok) ? &qkv_parts : nullptr);
}

spa_status run_layer_after_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int layer_index,
                                const spa_layer* next, const spa_batch* b, int tok0, int n_tok, const WsLayout& W,
                                const Slot& s, hipStream_t st, TimingHook* th, bool fuse_head) {
  spa_status rc;
  float* x = b->x + (size_t)tok0 * m->hidden;
  int32_t* rec = b->topk_out ? b->topk_out + ((size_t)layer_index * b->batch + tok0) * m->top_k : nullptr;
  if ((rc = op_oproj_route(ctx, m, l, x, n_tok, s, rec, fuse_head, st, th))) return rc;
  return run_segment_b(ctx, m, l, layer_index, next, b, tok0, n_tok, W, s, true, st, th);
}

spa_status run_segment_b(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int layer_index,
                         const spa_layer* next, const spa_batch* b, int tok0, int n_tok, const WsLayout& W,
                         const Slot& s, bool with_router, hipStream_t st, TimingHook* th) {
  (void)W;
  spa_status rc;
  float* x = b->x + (size_t)tok0 * m->hidden;
  if (!with_router) {
    int32_t* rec = b->topk_out ? b->topk_out + ((size_t)layer_index * b->batch + tok0) * m->top_k : nullptr;
    if ((rc = op_route(ctx, m, l, s.hn_f32, n_tok, s.logits, s.route, rec, s, st, th, route_gathers(m))))
      return rc;
  }
  // the router's permutation kernel gathered the expert rows, or left them in place (route_gathers)
  if ((rc = op_comm(ctx, m, s.xe_perm, (size_t)n_tok * m->top_k * m->hidden * esz_of(m->expert_dtype),
                     comm_bytes_dispatch(m, n_tok), s, st, th))) return rc;   // MoE dispatch
  GemmPlan dp{};
  if ((rc = op_expert(ctx, m, l, expert_input(m, s), s.hn8_scale, n_tok, s.route, s.y, s, st, th, &dp,
                      route_gathers(m) ? ExpertRows::kGathered : ExpertRows::kInPlace)))
    return rc;
  const size_t cb = comm_bytes_combine(m, n_tok);
  if ((rc = op_comm(ctx, m, s.y, cb, cb, s, st, th))) return rc;   // MoE combine
  const bool plain = dp.epi == EPI_STORE;
  return op_combine(m, s.h, plain ? s.y : nullptr, plain ? nullptr : &dp, &s, s.route, n_tok, x,
                    next ? next->gamma1 : nullptr, s.xn, st, th, true);
}

// ---------------------------------------------------------------------------
// argument checks
// ---------------------------------------------------------------------------
static spa_status check_batch(const spa_batch* b) {
  if (!b) return fail(SPA_EINVAL, "batch is NULL");
  if (b->batch < 1) return fail(SPA_EINVAL, "batch must be >= 1");
  if (b->max_kv_len < 1) return fail(SPA_EINVAL, "max_kv_len must be >= 1");
  if (!b->kv_len || !b->kv_off || !b->kv_cap || !b->x) return fail(SPA_EINVAL, "batch pointer is NULL");
  if (((uintptr_t)b->x) & 15) return fail(SPA_EINVAL, "x must be 16-byte aligned");
  return SPA_OK;
}

spa_status check_layer(const spa_model_desc* m, const spa_layer* l) {
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

spa_status check_tokens(const spa_model_desc* m, int n_tok) {
  if (n_tok < 1) return fail(SPA_EINVAL, "n_tok must be >= 1");
  if ((long long)n_tok * m->top_k > 4096) return fail(SPA_EUNSUPPORTED, "tokens * top_k above 4096 per microbatch");
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

static bool misaligned(const void* p) { return ((uintptr_t)p) & 15; }

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
  if (hipError_t ka = init_kernel_attributes()) {
    delete c;
    return hip_fail(ka, "kernel attributes");
  }
  if (spa_status rc = noalloc_bind_device(hip_device)) {
    delete c;
    return rc;
  }
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, hip_device) == hipSuccess && khz > 0)
    c->wall_khz = khz;
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
  if ((rc = check_tokens(m, batch / n_micro))) return rc;
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
  return clear_errors(ws, (hipStream_t)stream);
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
  a.kv_off = (const long long*)b->kv_off;
  a.kv_cap = b->kv_cap;
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

size_t spa_packed_bytes(int32_t dtype, int32_t n_mats, int32_t n_rows, int32_t k) {
  if (dtype != SPA_F32 && dtype != SPA_BF16 && dtype != SPA_E4M3) return 0;
  if (n_mats < 1 || n_rows < 1 || k < 1 || ((size_t)k * esz_of(dtype)) % 64) return 0;
  return (size_t)n_mats * ((size_t)(n_rows + 15) / 16 * 16) * k * esz_of(dtype);
}

spa_status spa_pack_weights(spa_ctx* ctx, int32_t dtype, int32_t n_mats, int32_t n_rows, int32_t k, const void* src,
                            void* dst, void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  if (dtype != SPA_F32 && dtype != SPA_BF16 && dtype != SPA_E4M3) return fail(SPA_EINVAL, "bad dtype");
  if (n_mats < 1 || n_rows < 1 || k < 1) return fail(SPA_EINVAL, "n_mats, n_rows and k must be >= 1");
  if (((size_t)k * esz_of(dtype)) % 64) return fail(SPA_EINVAL, "a row must be a whole number of 64-byte k-steps");
  if (!src || !dst || misaligned(src) || misaligned(dst)) return fail(SPA_EINVAL, "src/dst NULL or not 16-byte aligned");
  const size_t nb = spa_packed_bytes(dtype, n_mats, n_rows, k);
  const char *s0 = (const char*)src, *d0 = (const char*)dst;
  if (s0 < d0 + nb && d0 < s0 + (size_t)n_mats * n_rows * k * esz_of(dtype))
    return fail(SPA_EINVAL, "src and dst overlap");
  SPA_HIP(launch_pack_panels(src, dst, n_mats, n_rows, k, esz_of(dtype), (hipStream_t)stream));
  return SPA_OK;
}

spa_status spa_rms_norm(spa_ctx* ctx, const spa_model_desc* m, const float* x, const float* gamma, int32_t n_tok,
                        void* xn_out, void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if (!x || !gamma || !xn_out || n_tok < 1) return fail(SPA_EINVAL, "bad argument");
  spa_route_bufs none{};
  // combine with no expert terms: x is rewritten with itself, xn = RMSNorm(x) gamma
  return op_combine(m, x, nullptr, nullptr, nullptr, none, n_tok, const_cast<float*>(x), gamma, xn_out,
                    (hipStream_t)stream, nullptr);
}

#define SPA_OP_PROLOGUE(n_tok_expr)                                             \
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");                             \
  spa_status rc = validate_model(m);                                            \
  if (rc) return rc;                                                            \
  if ((rc = check_tokens(m, (n_tok_expr)))) return rc;                          \
  WsLayout W;                                                                   \
  if ((rc = check_ws(m, (n_tok_expr), max_kv, 1, ws, ws_bytes, &W))) return rc; \
  Slot s = slot_ptrs(W, ws, 0);                                                 \
  hipStream_t st = (hipStream_t)stream;                                         \
  if ((rc = clear_errors(ws, st))) return rc;

spa_status spa_qkv_append(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int32_t tok0,
                          int32_t n_tok, const void* xn, void* q_out, void* ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_batch(b);
  if (rc0) return rc0;
  if ((rc0 = check_layer(m, l))) return rc0;
  if (tok0 < 0 || n_tok < 1 || tok0 + n_tok > b->batch) return fail(SPA_EINVAL, "token range outside the batch");
  if (!xn || !q_out || misaligned(xn) || misaligned(q_out)) return fail(SPA_EINVAL, "xn / q_out NULL or misaligned");
  const int max_kv = b->max_kv_len;
  SPA_OP_PROLOGUE(n_tok)
  return op_qkv(ctx, m, l, b, tok0, n_tok, xn, q_out, s, st, nullptr);
}

spa_status spa_decode_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int32_t tok0,
                           int32_t n_tok, const void* q, void* o_out, void* ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_batch(b);
  if (rc0) return rc0;
  if ((rc0 = check_layer(m, l))) return rc0;
  if (tok0 < 0 || n_tok < 1 || tok0 + n_tok > b->batch) return fail(SPA_EINVAL, "token range outside the batch");
  if (!q || !o_out || misaligned(q)) return fail(SPA_EINVAL, "q / o_out NULL or misaligned");
  const int max_kv = b->max_kv_len;
  SPA_OP_PROLOGUE(n_tok)
  return op_attn(ctx, m, l, b, tok0, n_tok, q, o_out, W, s, st, nullptr);
}

}  // extern "C"

namespace spa {

// The attention operator on scratch the caller hands over (the no-allocation
// entry point's fixed device array): the chunk partials at part, the error
// word at err (cleared here unless the caller gave its own). The partial
// buffer holds exactly the chunks this call's shapes produce.
size_t attn_scratch_bytes(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int n_tok,
                          int* max_chunks_out) {
  const int G = m->n_q_heads / m->n_kv_heads;
  const int chunks = l->kind == SPA_FULL ? (b->max_kv_len + attn_chunk(m, b, n_tok, ctx->n_cus) - 1) /
                                               attn_chunk(m, b, n_tok, ctx->n_cus)
                                         : (m->window + kAttnChunk - 1) / kAttnChunk;
  if (max_chunks_out) *max_chunks_out = chunks;
  if (dealt_launch(l, n_tok)) return deal_part_bytes(deal_ranges(ctx->n_cus), n_tok, m->n_kv_heads, G, m->head_dim);
  return (size_t)n_tok * m->n_kv_heads * chunks * G * (m->head_dim + 2) * 4;
}

spa_status decode_attn_on_scratch(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b,
                                  int tok0, int n_tok, const void* q, void* o, float* part, size_t part_bytes,
                                  int32_t* err_word, bool clear_err, hipStream_t st) {
  int chunks = 0;
  const size_t need = attn_scratch_bytes(ctx, m, l, b, n_tok, &chunks);
  if (need > part_bytes)
    return fail(SPA_EWORKSPACE, "attention partials need " + std::to_string(need) + " bytes, the fixed scratch holds " +
                                    std::to_string(part_bytes));
  WsLayout W{};
  W.max_chunks = chunks;
  Slot s{};
  s.attn_part = part;
  s.err = err_word;
  if (clear_err) SPA_HIP(launch_fill_i32(err_word, 1, 0, st));
  return op_attn(ctx, m, l, b, tok0, n_tok, q, o, W, s, st, nullptr);
}

spa_status check_decode_attn_args(const spa_model_desc* m, const spa_layer* l, const spa_batch* b, int tok0, int n_tok,
                                  const void* q, const void* o_out) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if ((rc = check_batch(b))) return rc;
  if ((rc = check_layer(m, l))) return rc;
  if ((rc = check_tokens(m, n_tok))) return rc;
  if (tok0 < 0 || n_tok < 1 || tok0 + n_tok > b->batch) return fail(SPA_EINVAL, "token range outside the batch");
  if (!q || !o_out || misaligned(q)) return fail(SPA_EINVAL, "q / o_out NULL or misaligned");
  return SPA_OK;
}

}  // namespace spa

extern "C" {

spa_status spa_out_proj(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* x, const void* o,
                        int32_t n_tok, float* h_out, float* hn_out, void* ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_layer(m, l);
  if (rc0) return rc0;
  if (!x || !o || !h_out || !hn_out) return fail(SPA_EINVAL, "NULL pointer");
  if (misaligned(x) || misaligned(o) || misaligned(h_out) || misaligned(hn_out)) return fail(SPA_EINVAL, "misaligned tensor");
  const int max_kv = 1;
  SPA_OP_PROLOGUE(n_tok)
  return op_oproj(ctx, m, l, x, o, n_tok, h_out, hn_out, nullptr, nullptr, nullptr, s, st, nullptr);
}

spa_status spa_moe_route(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* hn, int32_t n_tok,
                         float* logits_out, const spa_route_bufs* r, int32_t* topk_rec, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_layer(m, l);
  if (rc0) return rc0;
  if (!hn || !logits_out || !r || misaligned(hn)) return fail(SPA_EINVAL, "bad argument");
  if (!r->topk_idx || !r->topk_w || !r->offsets || !r->row_tok || !r->row_slot || !r->inv)
    return fail(SPA_EINVAL, "route buffer is NULL");
  const int max_kv = 1;
  SPA_OP_PROLOGUE(n_tok)
  return op_route(ctx, m, l, hn, n_tok, logits_out, *r, topk_rec, s, st, nullptr);
}

spa_status spa_moe_expert(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* hn, int32_t n_tok,
                          const spa_route_bufs* r, float* y_out, void* ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_layer(m, l);
  if (rc0) return rc0;
  if (!hn || !r || !y_out || misaligned(hn) || !r->offsets || !r->row_tok) return fail(SPA_EINVAL, "bad argument");
  const int max_kv = 1;
  SPA_OP_PROLOGUE(n_tok)
  const void* xe = hn;
  if (m->expert_dtype != SPA_F32) {   // the expert input format of hn
    CvtArgs c;
    memset(&c, 0, sizeof(c));
    c.x = hn;
    c.n_rows = n_tok;
    c.n_cols = m->hidden;
    c.dtype = m->expert_dtype == SPA_BF16 ? DT_BF16 : DT_E4M3;
    c.out = m->expert_dtype == SPA_BF16 ? (void*)s.hn_bf16 : (void*)s.hn8;
    c.scales = s.hn8_scale;
    c.n_cus = ctx->n_cus;
    SPA_HIP(launch_cvt_rows(c, st));
    xe = c.out;
  }
  GemmPlan dp{};
  if ((rc = op_expert(ctx, m, l, xe, s.hn8_scale, n_tok, *r, y_out, s, st, nullptr, &dp))) return rc;
  if (dp.epi == EPI_PARTIAL) {
    CombineArgs a = combine_args(m, nullptr, nullptr, &dp, &s, *r, n_tok, y_out, nullptr, nullptr);
    SPA_HIP(launch_part_rows(a, n_tok * m->top_k, st));
  }
  return SPA_OK;
}

spa_status spa_moe_combine(spa_ctx* ctx, const spa_model_desc* m, const float* h, const float* y,
                           const spa_route_bufs* r, int32_t n_tok, float* x_out, const float* gamma_next, void* xn_out,
                           void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if (!h || !y || !r || !x_out || n_tok < 1) return fail(SPA_EINVAL, "bad argument");
  if (gamma_next && !xn_out) return fail(SPA_EINVAL, "xn_out needed with gamma_next");
  return op_combine(m, h, y, nullptr, nullptr, *r, n_tok, x_out, gamma_next, xn_out, (hipStream_t)stream, nullptr);
}

spa_status spa_virtual_comm(spa_ctx* ctx, const void* src, void* dst, size_t bytes, float latency_us, float gbps,
                            void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  if (bytes % 16 || bytes > ((size_t)1 << 32)) return fail(SPA_EINVAL, "bytes must be a multiple of 16, at most 2^32");
  if (bytes && (!src || !dst || misaligned(src) || misaligned(dst)))
    return fail(SPA_EINVAL, "src and dst must be 16-byte aligned device pointers");
  if (bytes && (const char*)src < (const char*)dst + bytes && (const char*)dst < (const char*)src + bytes)
    return fail(SPA_EINVAL, "src and dst overlap");
  if (!(latency_us >= 0.f) || !(gbps >= 0.f) || (bytes && gbps == 0.f))
    return fail(SPA_EINVAL, "latency_us must be >= 0 and gbps > 0");
  return launch_comm(ctx, src, dst, bytes, bytes, latency_us, gbps, (hipStream_t)stream);
}

spa_status spa_layer_forward(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int32_t layer_index,
                             const spa_batch* b, int32_t tok0, int32_t n_tok, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!m) return fail(SPA_EINVAL, "model is NULL");
  spa_status rc0 = check_batch(b);
  if (rc0) return rc0;
  if ((rc0 = check_layer(m, l))) return rc0;
  if (tok0 < 0 || n_tok < 1 || tok0 + n_tok > b->batch) return fail(SPA_EINVAL, "token range outside the batch");
  if (layer_index < 0 || layer_index >= m->n_layers) return fail(SPA_EINVAL, "layer_index out of range");
  const int max_kv = b->max_kv_len;
  SPA_OP_PROLOGUE(n_tok)
  if ((rc = run_segment_a(ctx, m, l, layer_index, nullptr, b, tok0, n_tok, W, s, true, true, st, nullptr, false)))
    return rc;
  return run_segment_b(ctx, m, l, layer_index, nullptr, b, tok0, n_tok, W, s, true, st, nullptr);
}

spa_status spa_temporal_run(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* layers, const spa_batch* b,
                            int32_t n_micro, void* ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(SPA_EINVAL, "ctx is NULL");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if ((rc = check_batch(b))) return rc;
  if (!layers) return fail(SPA_EINVAL, "layers is NULL");
  for (int i = 0; i < m->n_layers; ++i)
    if ((rc = check_layer(m, &layers[i]))) return rc;
  if (n_micro < 1 || b->batch % n_micro) return fail(SPA_EINVAL, "n_micro must divide the batch");
  const int bm = b->batch / n_micro;
  if ((rc = check_tokens(m, bm))) return rc;
  WsLayout W;
  if ((rc = check_ws(m, bm, b->max_kv_len, n_micro, ws, ws_bytes, &W))) return rc;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = clear_errors(ws, st))) return rc;
  // the pipeline's dispatch order (layer, then microbatch), serialised on one stream
  for (int li = 0; li < m->n_layers; ++li) {
    const spa_layer* next = li + 1 < m->n_layers ? &layers[li + 1] : nullptr;
    for (int mu = 0; mu < n_micro; ++mu) {
      Slot s = slot_ptrs(W, ws, mu);
      if ((rc = run_segment_a(ctx, m, &layers[li], li, next, b, mu * bm, bm, W, s, true, li == 0, st, nullptr, false)))
        return rc;
      if ((rc = run_segment_b(ctx, m, &layers[li], li, next, b, mu * bm, bm, W, s, true, st, nullptr))) return rc;
    }
  }
  return SPA_OK;
}

}  // extern "C"
