// CU pools and the two-stage spatial pipeline (sections 3.1-3.2 and 5.3.2 of
// the SubGPU Pipelining paper, realised with CU-masked HIP streams and
// events instead of Green Contexts).
#include <string.h>

#include <algorithm>
#include <set>
#include <string>
#include <vector>

#include <hip/hip_ext.h>

#include "host.h"

using namespace spa;

struct spa_pool {
  spa_ctx* ctx = nullptr;
  std::vector<uint32_t> mask;
  hipStream_t stream = nullptr;
  unsigned* probe_buf = nullptr;
};

struct spa_pipeline {
  spa_ctx* ctx = nullptr;
  spa_model_desc m{};
  spa_pipeline_cfg cfg{};
  spa_pool* a = nullptr;   // null: temporal (everything on the caller stream)
  spa_pool* b = nullptr;
  spa_pool* ak[2] = {nullptr, nullptr};   // stage pools per layer kind (spa_layer_kind)
  spa_pool* bk[2] = {nullptr, nullptr};
  std::vector<hipEvent_t> ev_end;         // one per distinct pool stream
  std::vector<hipEvent_t> evA, evB;   // [layer][micro] (hand-offs when stream value waits are unavailable)
  hipEvent_t ev_start = nullptr, ev_end_a = nullptr, ev_end_b = nullptr;
  // Hand-off counters in device memory: done_a[micro], done_b[micro]. The
  // stage that finishes (layer l, microbatch j) of run r writes r*n_layers +
  // l + 1 from its stream, the other stage's stream waits until the counter
  // reaches it; values only grow, so nothing is ever reset.
  uint64_t* flags = nullptr;
  uint64_t runs = 0;
  bool value_sync = false;
  int timed_cls = -1;
  int timed_mode = 0;                 // 1: device-clock spans for attention, 2: events
  std::vector<hipEvent_t> tevs, tpool;
  unsigned long long* tspan = nullptr;   // [kSpanCap][kSpanWords] device-clock spans
  unsigned long long* tspan_host = nullptr;   // pinned copy for the harvest
  int tspan_used = 0;
  double t_sum_ms = 0.0;
  int t_count = 0;
  // graph replay of temporal iterations (cfg.graph)
  hipStream_t gstream = nullptr;
  hipGraphExec_t gexec = nullptr;
  std::vector<unsigned char> gkey;      // the arguments the captured launches were built from
  hipEvent_t gev_in = nullptr, gev_out = nullptr;
  unsigned long long* gacc = nullptr;   // device: attention span ticks and launch count of replays
};

static constexpr int kSpanCap = 8192;   // timed launches between two harvests

static spa_status make_pool(spa_ctx* ctx, const std::vector<uint32_t>& mask, spa_pool** out) {
  int nbits = 0;
  for (size_t w = 0; w < mask.size(); ++w) {
    for (int bit = 0; bit < 32; ++bit) {
      if (mask[w] >> bit & 1u) {
        if ((int)(w * 32 + bit) >= ctx->n_cus) return fail(SPA_EMASK, "CU mask names a CU beyond the device");
        ++nbits;
      }
    }
  }
  if (nbits == 0) return fail(SPA_EMASK, "CU mask is empty");
  // runtime mask bit i runs on XCD i % n_xcd; the runtime refuses a mask that
  // leaves an XCD without CUs, so refuse it here before touching HIP
  for (int x = 0; x < ctx->n_xcd; ++x) {
    bool any = false;
    for (int bit = x; bit < ctx->n_cus && !any; bit += ctx->n_xcd)
      any = (size_t)(bit / 32) < mask.size() && (mask[bit / 32] >> (bit % 32) & 1u);
    if (!any) return fail(SPA_EMASK, "CU mask leaves XCD " + std::to_string(x) + " without CUs");
  }
  spa_pool* p = new spa_pool();
  p->ctx = ctx;
  p->mask = mask;
  hipError_t e = hipSetDevice(ctx->device);
  if (e == hipSuccess) e = hipExtStreamCreateWithCUMask(&p->stream, (uint32_t)mask.size(), mask.data());
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete p;
    return hip_fail(e, "hipExtStreamCreateWithCUMask");
  }
  register_stream_cus(p->stream, nbits);
  *out = p;
  return SPA_OK;
}

// Distinct hardware CUs (packed ids) that n_blocks short workgroups on the
// pool's stream ran on.
static spa_status probe_ids(spa_pool* p, int n_blocks, std::set<uint32_t>* ids) {
  unsigned* buf = nullptr;
  SPA_HIP(hipMalloc(&buf, sizeof(unsigned) * 2 * n_blocks));
  std::vector<unsigned> h(2 * (size_t)n_blocks);
  hipError_t e = launch_probe(buf, n_blocks, 20000, p->stream);
  if (e == hipSuccess) e = hipMemcpyAsync(h.data(), buf, h.size() * sizeof(unsigned), hipMemcpyDeviceToHost, p->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(p->stream);
  (void)hipFree(buf);
  if (e != hipSuccess) return hip_fail(e, "probe");
  for (int i = 0; i < n_blocks; ++i) {
    unsigned xcc = h[2 * i] & 0xF, hw = h[2 * i + 1];
    unsigned cu = (hw >> 8) & 0xF, sh = (hw >> 12) & 1, se = (hw >> 13) & 7;
    ids->insert((xcc << 16) | (se << 8) | (sh << 4) | cu);
  }
  return SPA_OK;
}

extern "C" {

spa_status spa_pool_create_mask(spa_ctx* ctx, const uint32_t* cu_mask, int32_t n_words, spa_pool** out) {
  if (!ctx || !cu_mask || !out || n_words < 1) return fail(SPA_EINVAL, "bad argument");
  std::vector<uint32_t> m(cu_mask, cu_mask + n_words);
  return make_pool(ctx, m, out);
}

spa_status spa_pool_create_split(spa_ctx* ctx, int32_t first_per_xcd, int32_t n_cus, spa_pool** out) {
  if (!ctx || !out) return fail(SPA_EINVAL, "bad argument");
  const int nx = ctx->n_xcd;
  const int per_xcd = ctx->n_cus / nx;
  if (n_cus < nx || n_cus % nx) return fail(SPA_EINVAL, "n_cus must be a positive multiple of the XCD count");
  const int take = n_cus / nx;
  if (first_per_xcd < 0 || first_per_xcd + take > per_xcd) return fail(SPA_EINVAL, "CU range beyond an XCD");
  // runtime CU mask bit i belongs to XCD i % n_xcd (mask bits are dealt to
  // the XCDs round-robin); its index inside the XCD is i / n_xcd
  std::vector<uint32_t> mask((ctx->n_cus + 31) / 32, 0u);
  for (int x = 0; x < nx; ++x)
    for (int j = first_per_xcd; j < first_per_xcd + take; ++j) {
      int bit = j * nx + x;
      mask[bit / 32] |= 1u << (bit % 32);
    }
  return make_pool(ctx, mask, out);
}

spa_status spa_pool_mask(spa_pool* p, uint32_t* mask_out, int32_t n_words) {
  if (!p || !mask_out) return fail(SPA_EINVAL, "bad argument");
  for (int i = 0; i < n_words; ++i) mask_out[i] = i < (int)p->mask.size() ? p->mask[i] : 0u;
  return SPA_OK;
}

spa_status spa_pool_stream(spa_pool* p, void** s) {
  if (!p || !s) return fail(SPA_EINVAL, "bad argument");
  *s = (void*)p->stream;
  return SPA_OK;
}

spa_status spa_pool_probe(spa_pool* p, int32_t n_blocks, uint32_t* ids_out, int32_t max_ids, int32_t* n_ids) {
  if (!p || !ids_out || !n_ids || n_blocks < 1 || n_blocks > (1 << 20)) return fail(SPA_EINVAL, "bad argument");
  std::set<uint32_t> ids;
  spa_status rc = probe_ids(p, n_blocks, &ids);
  if (rc) return rc;
  int n = 0;
  for (uint32_t v : ids) {
    if (n < max_ids) ids_out[n] = v;
    ++n;
  }
  *n_ids = n;
  return SPA_OK;
}

spa_status spa_pool_verify(spa_pool* p, int32_t* observed_out) {
  if (!p) return fail(SPA_EINVAL, "bad argument");
  const int nx = p->ctx->n_xcd;
  std::vector<int> want(nx, 0);
  int n_mask = 0;
  for (size_t w = 0; w < p->mask.size(); ++w)
    for (int bit = 0; bit < 32; ++bit)
      if (p->mask[w] >> bit & 1u) {
        ++want[(w * 32 + bit) % nx];
        ++n_mask;
      }
  std::set<uint32_t> ids;
  spa_status rc = probe_ids(p, std::min(1 << 16, 64 * n_mask), &ids);
  if (rc) return rc;
  std::vector<int> got(16, 0);
  for (uint32_t v : ids) ++got[(v >> 16) & 0xF];
  if (observed_out) *observed_out = (int32_t)ids.size();
  // XCD labels of the hardware ids need not follow the mask's numbering:
  // compare the per-XCD counts as sorted lists
  std::vector<int> g(got.begin(), got.end()), wnt(want.begin(), want.end());
  g.erase(std::remove(g.begin(), g.end(), 0), g.end());
  wnt.erase(std::remove(wnt.begin(), wnt.end(), 0), wnt.end());
  std::sort(g.begin(), g.end());
  std::sort(wnt.begin(), wnt.end());
  const bool over = (int)ids.size() > n_mask || g.size() > wnt.size();
  bool per_xcd_over = false;
  if (!over && g.size() == wnt.size())
    for (size_t i = 0; i < g.size(); ++i) per_xcd_over |= g[i] > wnt[i];
  if (over || per_xcd_over || g.size() != wnt.size())
    return fail(SPA_EMASK, "pool kernels ran on " + std::to_string(ids.size()) + " CUs over " +
                               std::to_string(g.size()) + " XCDs; the mask holds " + std::to_string(n_mask) +
                               " CUs over " + std::to_string(wnt.size()) + " XCDs");
  return SPA_OK;
}

spa_status spa_pool_destroy(spa_pool* p) {
  if (!p) return SPA_OK;
  if (p->stream) {
    unregister_stream_cus(p->stream);
    (void)hipStreamDestroy(p->stream);
  }
  delete p;
  return SPA_OK;
}

static bool pools_overlap(const spa_pool* x, const spa_pool* y) {
  const size_t nw = std::max(x->mask.size(), y->mask.size());
  for (size_t w = 0; w < nw; ++w) {
    const uint32_t mx = w < x->mask.size() ? x->mask[w] : 0u;
    const uint32_t my = w < y->mask.size() ? y->mask[w] : 0u;
    if (mx & my) return true;
  }
  return false;
}

static spa_status create_impl(spa_ctx* ctx, const spa_model_desc* m, const spa_pipeline_cfg* cfg, spa_pool* a_full,
                              spa_pool* b_full, spa_pool* a_slide, spa_pool* b_slide, spa_pipeline** out) {
  if (!ctx || !cfg || !out) return fail(SPA_EINVAL, "bad argument");
  spa_status rc = validate_model(m);
  if (rc) return rc;
  if (cfg->cut < 0 || cfg->cut > 2) return fail(SPA_EINVAL, "cut must be 0, 1 or 2");
  if (cfg->n_micro < 1) return fail(SPA_EINVAL, "n_micro must be >= 1");
  if (cfg->handoff != 0 && cfg->handoff != 1) return fail(SPA_EINVAL, "handoff must be 0 (value waits) or 1 (events)");
  if (cfg->graph != 0 && cfg->graph != 1) return fail(SPA_EINVAL, "graph must be 0 or 1");
  if (cfg->head != 0 && cfg->head != 1) return fail(SPA_EINVAL, "head must be 0 (separate launches) or 1 (one launch)");
  if (cfg->graph && (a_full || b_full || a_slide || b_slide))
    return fail(SPA_EUNSUPPORTED, "graph replay needs the temporal schedule: graph kernel nodes do not keep a CU mask");
  const bool any = a_full || b_full || a_slide || b_slide;
  const bool all = a_full && b_full && a_slide && b_slide;
  if (any && !all) return fail(SPA_EINVAL, "give both pools of every layer kind, or none");
  if (all) {
    if (a_full == b_full || a_slide == b_slide) return fail(SPA_EMASK, "the two stages need distinct pools");
    if (pools_overlap(a_full, b_full) || pools_overlap(a_slide, b_slide)) return fail(SPA_EMASK, "stage CU pools overlap");
  }
  spa_pipeline* p = new spa_pipeline();
  p->ctx = ctx;
  p->m = *m;
  p->cfg = *cfg;
  p->a = a_full;
  p->b = b_full;
  p->ak[SPA_FULL] = a_full;
  p->bk[SPA_FULL] = b_full;
  p->ak[SPA_SLIDING] = a_slide;
  p->bk[SPA_SLIDING] = b_slide;
  const size_t n_ev = (size_t)m->n_layers * cfg->n_micro;
  p->evA.resize(n_ev, nullptr);
  p->evB.resize(n_ev, nullptr);
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < n_ev && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&p->evA[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->evB[i], hipEventDisableTiming);
  }
  if (e == hipSuccess && all) {
    e = hipMalloc(&p->flags, sizeof(uint64_t) * 2 * cfg->n_micro);
    if (e == hipSuccess) e = hipMemset(p->flags, 0, sizeof(uint64_t) * 2 * cfg->n_micro);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess && cfg->handoff == 0) {
      // use stream value writes/waits when the runtime supports them on this memory
      hipError_t t = hipStreamWriteValue64(a_full->stream, p->flags, 0, 0);
      if (t == hipSuccess) t = hipStreamWaitValue64(b_full->stream, p->flags, 0, hipStreamWaitValueGte, ~0ull);
      if (t == hipSuccess) t = hipDeviceSynchronize();
      p->value_sync = t == hipSuccess;
      if (t != hipSuccess) (void)hipGetLastError();
    }
    // one join event per distinct stream
    std::vector<hipStream_t> seen;
    for (spa_pool* q : {a_full, b_full, a_slide, b_slide})
      if (std::find(seen.begin(), seen.end(), q->stream) == seen.end()) seen.push_back(q->stream);
    p->ev_end.resize(seen.size(), nullptr);
    for (size_t i = 0; i < seen.size() && e == hipSuccess; ++i)
      e = hipEventCreateWithFlags(&p->ev_end[i], hipEventDisableTiming);
  }
  if (e == hipSuccess && cfg->graph) {
    e = hipStreamCreateWithFlags(&p->gstream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->gev_in, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->gev_out, hipEventDisableTiming);
    if (e == hipSuccess) e = hipMalloc(&p->gacc, 2 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMemset(p->gacc, 0, 2 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_start, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_end_a, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ev_end_b, hipEventDisableTiming);
  if (e != hipSuccess) {
    spa_pipeline_destroy(p);
    return hip_fail(e, "hipEventCreate");
  }
  *out = p;
  return SPA_OK;
}

spa_status spa_pipeline_create(spa_ctx* ctx, const spa_model_desc* m, const spa_pipeline_cfg* cfg, spa_pool* stage_a,
                               spa_pool* stage_b, spa_pipeline** out) {
  if ((stage_a == nullptr) != (stage_b == nullptr)) return fail(SPA_EINVAL, "give both pools or neither");
  return create_impl(ctx, m, cfg, stage_a, stage_b, stage_a, stage_b, out);
}

spa_status spa_pipeline_create_kinds(spa_ctx* ctx, const spa_model_desc* m, const spa_pipeline_cfg* cfg,
                                     spa_pool* a_full, spa_pool* b_full, spa_pool* a_sliding, spa_pool* b_sliding,
                                     spa_pipeline** out) {
  return create_impl(ctx, m, cfg, a_full, b_full, a_sliding, b_sliding, out);
}

// Clears span slots [0, n) (zero: no start stored, identity of the atomic max).
static hipError_t reset_spans(spa_pipeline* p, int n) {
  if (n <= 0) return hipSuccess;
  hipError_t e = launch_fill_i32((int*)p->tspan, (long long)n * kSpanWords * 2, 0, nullptr);
  return e == hipSuccess ? hipDeviceSynchronize() : e;
}

static spa_status harvest_timing(spa_pipeline* p) {
  if (p->gacc) {   // graph replays: spans folded on the device by the graph's last kernel
    unsigned long long acc[2] = {0, 0};
    SPA_HIP(hipMemcpy(acc, p->gacc, sizeof(acc), hipMemcpyDeviceToHost));
    if (acc[1] > 0) {
      int khz = 0;
      SPA_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, p->ctx->device));
      if (khz <= 0) return fail(SPA_EHIP, "device wall clock rate unknown");
      p->t_sum_ms += (double)acc[0] / khz;
      p->t_count += (int)acc[1];
      SPA_HIP(hipMemset(p->gacc, 0, sizeof(acc)));
      SPA_HIP(hipDeviceSynchronize());
    }
  }
  if (p->tspan_used > 0) {
    // spans: first workgroup start to last workgroup end, in wall-clock ticks
    int khz = 0;
    SPA_HIP(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, p->ctx->device));
    if (khz <= 0) return fail(SPA_EHIP, "device wall clock rate unknown");
    SPA_HIP(hipMemcpy(p->tspan_host, p->tspan, (size_t)kSpanWords * p->tspan_used * sizeof(unsigned long long),
                      hipMemcpyDeviceToHost));
    for (int i = 0; i < p->tspan_used; ++i) {
      const unsigned long long* w = p->tspan_host + (size_t)kSpanWords * i;
      unsigned long long end = 0;
      for (int j = 1; j <= 16; ++j) end = std::max(end, w[8 * j]);
      if (w[0] == 0 || end < w[0]) continue;   // a launch that did no timed work
      p->t_sum_ms += (double)(end - w[0]) / khz;
      p->t_count += 1;
    }
    SPA_HIP(reset_spans(p, p->tspan_used));
    p->tspan_used = 0;
  }
  // pairs (start, stop) in launch order; all complete once the caller synchronised
  for (size_t i = 0; i + 1 < p->tevs.size(); i += 2) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p->tevs[i], p->tevs[i + 1]) == hipSuccess) {
      p->t_sum_ms += ms;
      p->t_count += 1;
    }
    p->tpool.push_back(p->tevs[i]);
    p->tpool.push_back(p->tevs[i + 1]);
  }
  p->tevs.clear();
  return SPA_OK;
}

// Whether the MoE head runs as one persistent launch: asked for, and its
// workgroups wait for each other, so no other such launch may compete for
// the same CUs - true when every stage has one pool (a stream runs its tasks
// one at a time and the stages' pools are disjoint) or the schedule is
// temporal.
static bool head_fusable(const spa_pipeline* p) {
  if (p->cfg.head != 1) return false;
  return p->a == nullptr || (p->ak[SPA_FULL] == p->ak[SPA_SLIDING] && p->bk[SPA_FULL] == p->bk[SPA_SLIDING]);
}

// The Macro cut (P1 section 5.3.2): stage A runs only the full-attention
// launches; stage B runs everything else. For each full layer F, microbatch
// mu's stage-B segment is: what follows the previous full layer's attention
// (output projection .. combine), every sliding layer in between, and F's
// Norm+QKV; A(F, mu) waits for that segment, the next segment of mu waits for
// A(F, mu). Hand-off values: base + F + 1 for full layer F.
static spa_status run_macro(spa_pipeline* p, const spa_layer* layers, const spa_batch* b, void* ws,
                            const WsLayout& W, int bm, TimingHook* thp, uint64_t base) {
  const spa_model_desc* m = &p->m;
  const int n_micro = p->cfg.n_micro, L = m->n_layers;
  const hipStream_t sa = p->ak[SPA_FULL]->stream, sb = p->bk[SPA_FULL]->stream;
  const bool vs = p->value_sync;
  uint64_t* done_a = p->flags;
  uint64_t* done_b = p->flags ? p->flags + n_micro : nullptr;
  auto next_of = [&](int l) { return l + 1 < L ? &layers[l + 1] : nullptr; };
  spa_status rc;
  int prev = -1;   // the previous full layer
  for (int F = 0; F <= L; ++F) {
    const bool end = F == L;
    if (!end && layers[F].kind != SPA_FULL) continue;
    for (int mu = 0; mu < n_micro; ++mu) {
      const Slot s = slot_ptrs(W, ws, mu);
      const int tok0 = mu * bm;
      if (prev >= 0) {
        if (vs) SPA_HIP(hipStreamWaitValue64(sb, done_a + mu, base + (uint64_t)prev + 1, hipStreamWaitValueGte, ~0ull));
        else SPA_HIP(hipStreamWaitEvent(sb, p->evA[(size_t)prev * n_micro + mu], 0));
        if ((rc = run_layer_after_attn(p->ctx, m, &layers[prev], prev, next_of(prev), b, tok0, bm, W, s, sb, thp,
                                       head_fusable(p))))
          return rc;
      }
      for (int l = prev + 1; l < F; ++l) {   // the layers in between run whole on stage B
        if ((rc = run_layer_before_attn(p->ctx, m, &layers[l], b, tok0, bm, s, l == 0, sb, thp))) return rc;
        if ((rc = run_layer_attn(p->ctx, m, &layers[l], b, tok0, bm, W, s, sb, thp))) return rc;
        if ((rc = run_layer_after_attn(p->ctx, m, &layers[l], l, next_of(l), b, tok0, bm, W, s, sb, thp,
                                       head_fusable(p))))
          return rc;
      }
      if (end) continue;
      if ((rc = run_layer_before_attn(p->ctx, m, &layers[F], b, tok0, bm, s, F == 0, sb, thp))) return rc;
      if (vs) SPA_HIP(hipStreamWriteValue64(sb, done_b + mu, base + (uint64_t)F + 1, 0));
      else SPA_HIP(hipEventRecord(p->evB[(size_t)F * n_micro + mu], sb));
    }
    if (end) break;
    for (int mu = 0; mu < n_micro; ++mu) {
      const Slot s = slot_ptrs(W, ws, mu);
      if (vs) SPA_HIP(hipStreamWaitValue64(sa, done_b + mu, base + (uint64_t)F + 1, hipStreamWaitValueGte, ~0ull));
      else SPA_HIP(hipStreamWaitEvent(sa, p->evB[(size_t)F * n_micro + mu], 0));
      if ((rc = run_layer_attn(p->ctx, m, &layers[F], b, mu * bm, bm, W, s, sa, thp))) return rc;
      if (vs) SPA_HIP(hipStreamWriteValue64(sa, done_a + mu, base + (uint64_t)F + 1, 0));
      else SPA_HIP(hipEventRecord(p->evA[(size_t)F * n_micro + mu], sa));
    }
    prev = F;
  }
  return SPA_OK;
}

static spa_status enqueue_run(spa_pipeline* p, const spa_layer* layers, const spa_batch* b, void* ws,
                              const WsLayout& W, int bm, hipStream_t cs, TimingHook* thp);
static spa_status run_graph(spa_pipeline* p, const spa_layer* layers, const spa_batch* b, void* ws, size_t ws_bytes,
                            const WsLayout& W, int bm, hipStream_t cs);

spa_status spa_pipeline_run(spa_pipeline* p, const spa_layer* layers, const spa_batch* b, void* ws, size_t ws_bytes,
                            void* caller_stream) {
  if (!p || !layers || !b) return fail(SPA_EINVAL, "bad argument");
  const spa_model_desc* m = &p->m;
  const int n_micro = p->cfg.n_micro;
  if (b->batch < 1 || b->batch % n_micro) return fail(SPA_EINVAL, "n_micro must divide the batch");
  if (!b->x || !b->kv_len || !b->kv_off || !b->kv_cap || b->max_kv_len < 1) return fail(SPA_EINVAL, "bad batch");
  if ((long long)(b->batch / n_micro) * m->top_k > 4096) return fail(SPA_EUNSUPPORTED, "microbatch * top_k above 4096");
  for (int i = 0; i < m->n_layers; ++i) {
    const spa_layer* l = &layers[i];
    if (!l->wqkv || !l->wo || !l->wr || !l->wgu || !l->wd || !l->gamma1 || !l->gamma2 || !l->sinks || !l->k_cache ||
        !l->v_cache || (l->kind != SPA_FULL && l->kind != SPA_SLIDING))
      return fail(SPA_EINVAL, "incomplete layer " + std::to_string(i));
    if (m->expert_dtype == SPA_E4M3 && (!l->wgu_scale || !l->wd_scale))
      return fail(SPA_EINVAL, "E4M3 experts need scales");
  }
  const int bm = b->batch / n_micro;
  if (!ws || (((uintptr_t)ws) & 255)) return fail(SPA_EINVAL, "workspace NULL or not 256-byte aligned");
  WsLayout W = ws_layout(m, bm, b->max_kv_len, n_micro);
  if (ws_bytes < W.total) return fail(SPA_EWORKSPACE, "workspace too small: need " + std::to_string(W.total));

  hipStream_t cs = (hipStream_t)caller_stream;
  if (p->a == nullptr && p->cfg.graph && p->timed_mode != 2) return run_graph(p, layers, b, ws, ws_bytes, W, bm, cs);
  TimingHook th;
  th.cls = p->timed_cls;
  th.evs = &p->tevs;
  th.pool = &p->tpool;
  if (p->timed_mode == 1) {
    th.span = p->tspan;
    th.span_used = &p->tspan_used;
    th.span_cap = kSpanCap;
  }
  TimingHook* thp = p->timed_cls >= 0 ? &th : nullptr;
  return enqueue_run(p, layers, b, ws, W, bm, cs, thp);
}

// One iteration enqueued: temporal on cs, or spatial on the pools' streams
// joined to cs at both ends.
static spa_status enqueue_run(spa_pipeline* p, const spa_layer* layers, const spa_batch* b, void* ws,
                              const WsLayout& W, int bm, hipStream_t cs, TimingHook* thp) {
  const spa_model_desc* m = &p->m;
  const int n_micro = p->cfg.n_micro;
  spa_status rc = clear_errors(ws, cs);
  if (rc) return rc;
  const bool temporal = p->a == nullptr;
  // temporal: both segments share the stream, so the router may run in
  // segment A (where the output projection is) at no change to the results
  const bool router_in_a = temporal || p->cfg.cut == 1;
  const bool fuse = head_fusable(p);
  // stage streams of a layer (its kind's pools); the distinct streams for the joins
  auto stream_a = [&](const spa_layer* l) { return temporal ? cs : p->ak[l->kind == SPA_FULL ? SPA_FULL : SPA_SLIDING]->stream; };
  auto stream_b = [&](const spa_layer* l) { return temporal ? cs : p->bk[l->kind == SPA_FULL ? SPA_FULL : SPA_SLIDING]->stream; };
  std::vector<hipStream_t> streams;
  if (!temporal)
    for (spa_pool* q : {p->ak[SPA_FULL], p->bk[SPA_FULL], p->ak[SPA_SLIDING], p->bk[SPA_SLIDING]})
      if (std::find(streams.begin(), streams.end(), q->stream) == streams.end()) streams.push_back(q->stream);
  if (!temporal) {
    SPA_HIP(hipEventRecord(p->ev_start, cs));
    for (hipStream_t q : streams) SPA_HIP(hipStreamWaitEvent(q, p->ev_start, 0));
  }
  const bool vs = !temporal && p->value_sync;
  uint64_t* done_a = p->flags;
  uint64_t* done_b = p->flags ? p->flags + n_micro : nullptr;
  // a run that fails midway still consumes its values: the next run never
  // mistakes one of its writes for its own
  const uint64_t base = p->runs++ * (uint64_t)m->n_layers;
  if (!temporal && p->cfg.cut == 2) {
    rc = run_macro(p, layers, b, ws, W, bm, thp, base);
    if (rc) return rc;
    for (size_t i = 0; i < streams.size(); ++i) {
      SPA_HIP(hipEventRecord(p->ev_end[i], streams[i]));
      SPA_HIP(hipStreamWaitEvent(cs, p->ev_end[i], 0));
    }
    return SPA_OK;
  }
  for (int l = 0; l < m->n_layers; ++l) {
    const hipStream_t sa = stream_a(&layers[l]), sb = stream_b(&layers[l]);
    for (int mu = 0; mu < n_micro; ++mu) {
      Slot s = slot_ptrs(W, ws, mu);
      const size_t ei = (size_t)l * n_micro + mu;
      const uint64_t tick = base + (uint64_t)l + 1;   // hand-off value of (l, mu) in this run
      if (!temporal && l > 0) {
        if (vs) SPA_HIP(hipStreamWaitValue64(sa, done_b + mu, tick - 1, hipStreamWaitValueGte, ~0ull));
        else SPA_HIP(hipStreamWaitEvent(sa, p->evB[ei - n_micro], 0));
      }
      const spa_layer* next = l + 1 < m->n_layers ? &layers[l + 1] : nullptr;
      rc = run_segment_a(p->ctx, m, &layers[l], l, next, b, mu * bm, bm, W, s, router_in_a, l == 0, sa, thp, fuse);
      if (rc) return rc;
      if (vs) {
        SPA_HIP(hipStreamWriteValue64(sa, done_a + mu, tick, 0));
        SPA_HIP(hipStreamWaitValue64(sb, done_a + mu, tick, hipStreamWaitValueGte, ~0ull));
      } else if (!temporal) {
        SPA_HIP(hipEventRecord(p->evA[ei], sa));
        SPA_HIP(hipStreamWaitEvent(sb, p->evA[ei], 0));
      }
      rc = run_segment_b(p->ctx, m, &layers[l], l, next, b, mu * bm, bm, W, s, router_in_a, sb, thp);
      if (rc) return rc;
      if (vs) SPA_HIP(hipStreamWriteValue64(sb, done_b + mu, tick, 0));
      else if (!temporal) SPA_HIP(hipEventRecord(p->evB[ei], sb));
    }
  }
  if (!temporal) {
    for (size_t i = 0; i < streams.size(); ++i) {
      SPA_HIP(hipEventRecord(p->ev_end[i], streams[i]));
      SPA_HIP(hipStreamWaitEvent(cs, p->ev_end[i], 0));
    }
  }
  return SPA_OK;
}

// Everything a captured iteration's launches were built from.
static std::vector<unsigned char> graph_key(const spa_pipeline* p, const spa_layer* layers, const spa_batch* b,
                                            void* ws, size_t ws_bytes) {
  std::vector<unsigned char> k;
  auto put = [&](const void* x, size_t n) {
    const unsigned char* c = static_cast<const unsigned char*>(x);
    k.insert(k.end(), c, c + n);
  };
  put(layers, sizeof(spa_layer) * (size_t)p->m.n_layers);
  put(b, sizeof(*b));
  put(&ws, sizeof(ws));
  put(&ws_bytes, sizeof(ws_bytes));
  put(&p->timed_cls, sizeof(p->timed_cls));
  put(&p->timed_mode, sizeof(p->timed_mode));
  return k;
}

// Temporal iteration from a HIP graph: captured on the pipeline's own stream
// when the arguments differ from the last capture, then launched there
// between two event joins with the caller's stream. With the attention timer
// on (device-clock spans), the captured launches record into fixed slots and
// the graph's last kernel folds their spans into an accumulator and clears
// them, so every replay is timed inside the graph itself.
static spa_status run_graph(spa_pipeline* p, const spa_layer* layers, const spa_batch* b, void* ws, size_t ws_bytes,
                            const WsLayout& W, int bm, hipStream_t cs) {
  std::vector<unsigned char> key = graph_key(p, layers, b, ws, ws_bytes);
  if (!p->gexec || key != p->gkey) {
    if (p->gexec) {
      SPA_HIP(hipStreamSynchronize(p->gstream));
      (void)hipGraphExecDestroy(p->gexec);
      p->gexec = nullptr;
    }
    int n_spans = 0;
    TimingHook th;
    th.cls = p->timed_cls;
    th.evs = &p->tevs;
    th.pool = &p->tpool;
    if (p->timed_mode == 1) {
      th.span = p->tspan;
      th.span_used = &n_spans;
      th.span_cap = kSpanCap;
    }
    TimingHook* thp = p->timed_cls >= 0 ? &th : nullptr;
    SPA_HIP(hipStreamBeginCapture(p->gstream, hipStreamCaptureModeThreadLocal));
    spa_status rc = enqueue_run(p, layers, b, ws, W, bm, p->gstream, thp);
    if (!rc && n_spans > 0) {
      hipError_t e = launch_span_fold(p->tspan, n_spans, p->gacc, p->gstream);
      if (e != hipSuccess) rc = hip_fail(e, "span fold");
    }
    hipGraph_t g = nullptr;
    hipError_t ec = hipStreamEndCapture(p->gstream, &g);   // always end the capture
    if (!rc && ec != hipSuccess) rc = hip_fail(ec, "hipStreamEndCapture");
    if (!rc) {
      hipError_t ei = hipGraphInstantiate(&p->gexec, g, nullptr, nullptr, 0);
      if (ei != hipSuccess) {
        p->gexec = nullptr;
        rc = hip_fail(ei, "hipGraphInstantiate");
      }
    }
    if (g) (void)hipGraphDestroy(g);
    if (rc) {
      (void)hipGetLastError();
      return rc;
    }
    p->gkey = std::move(key);
  }
  SPA_HIP(hipEventRecord(p->gev_in, cs));
  SPA_HIP(hipStreamWaitEvent(p->gstream, p->gev_in, 0));
  SPA_HIP(hipGraphLaunch(p->gexec, p->gstream));
  SPA_HIP(hipEventRecord(p->gev_out, p->gstream));
  SPA_HIP(hipStreamWaitEvent(cs, p->gev_out, 0));
  return SPA_OK;
}

spa_status spa_pipeline_time_kernel(spa_pipeline* p, int32_t cls, int32_t enable) {
  if (!p || cls < 0 || cls >= KC_COUNT || enable < 0 || enable > 2) return fail(SPA_EINVAL, "bad argument");
  if (!p->tevs.empty() || p->tspan_used > 0) {
    SPA_HIP(hipDeviceSynchronize());
    spa_status rc = harvest_timing(p);
    if (rc) return rc;
  }
  const bool clock = enable == 1 && (cls == KC_ATTN_FULL || cls == KC_ATTN_SLIDING);
  if (clock && !p->tspan) {
    SPA_HIP(hipSetDevice(p->ctx->device));
    const size_t bytes = (size_t)kSpanCap * kSpanWords * sizeof(unsigned long long);
    hipError_t e = hipMalloc(&p->tspan, bytes);
    if (e == hipSuccess) e = hipHostMalloc(&p->tspan_host, bytes, hipHostMallocDefault);
    if (e == hipSuccess) e = reset_spans(p, kSpanCap);
    if (e != hipSuccess) {
      if (p->tspan) (void)hipFree(p->tspan);
      if (p->tspan_host) (void)hipHostFree(p->tspan_host);
      p->tspan = nullptr;
      p->tspan_host = nullptr;
      return hip_fail(e, "timing buffer");
    }
  }
  p->timed_cls = enable ? cls : -1;
  p->timed_mode = !enable ? 0 : clock ? 1 : 2;
  p->t_sum_ms = 0.0;
  p->t_count = 0;
  return SPA_OK;
}

spa_status spa_pipeline_timing(spa_pipeline* p, double* mean_ms, int32_t* count) {
  if (!p || !mean_ms || !count) return fail(SPA_EINVAL, "bad argument");
  SPA_HIP(hipDeviceSynchronize());
  spa_status rc = harvest_timing(p);
  if (rc) return rc;
  *count = p->t_count;
  *mean_ms = p->t_count ? p->t_sum_ms / p->t_count : 0.0;
  return SPA_OK;
}

spa_status spa_pipeline_destroy(spa_pipeline* p) {
  if (!p) return SPA_OK;
  (void)hipDeviceSynchronize();
  for (hipEvent_t e : p->evA)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->evB)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->tevs) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->tpool) (void)hipEventDestroy(e);
  if (p->tspan) (void)hipFree(p->tspan);
  if (p->tspan_host) (void)hipHostFree(p->tspan_host);
  if (p->flags) (void)hipFree(p->flags);
  for (hipEvent_t e : p->ev_end)
    if (e) (void)hipEventDestroy(e);
  if (p->gexec) (void)hipGraphExecDestroy(p->gexec);
  if (p->gstream) (void)hipStreamDestroy(p->gstream);
  if (p->gev_in) (void)hipEventDestroy(p->gev_in);
  if (p->gev_out) (void)hipEventDestroy(p->gev_out);
  if (p->gacc) (void)hipFree(p->gacc);
  if (p->ev_start) (void)hipEventDestroy(p->ev_start);
  if (p->ev_end_a) (void)hipEventDestroy(p->ev_end_a);
  if (p->ev_end_b) (void)hipEventDestroy(p->ev_end_b);
  delete p;
  return SPA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// tuner
namespace {

struct TuneCtx {
  spa_ctx* ctx;
  const spa_model_desc* m;
  const spa_layer* layers;
  const spa_batch* b;
  void* ws;
  size_t ws_bytes;
  const spa_tune_space* sp;
  hipStream_t st;
  hipEvent_t e0, e1;
  std::vector<spa_tune_point> points;
  spa_status err = SPA_OK;
  int cut = 0, n_micro = 1;
  int refine_kind = SPA_FULL, fixed_full = 0, fixed_slide = 0;
  bool per_kind = false;
};

// median time of reps iterations of one configuration (cu_a = 0: temporal)
spa_status measure(TuneCtx& t, int cut, int n_micro, int cu_full, int cu_slide, double* ms) {
  std::vector<spa_pool*> pools;
  spa_pipeline* pipe = nullptr;
  spa_status rc = SPA_OK;
  auto split = [&](int cu_a) {
    spa_pool *pa = nullptr, *pb = nullptr;
    if (!rc) rc = spa_pool_create_split(t.ctx, 0, cu_a, &pa);
    if (pa) pools.push_back(pa);
    if (!rc) rc = spa_pool_create_split(t.ctx, cu_a / t.ctx->n_xcd, t.ctx->n_cus - cu_a, &pb);
    if (pb) pools.push_back(pb);
  };
  spa_pipeline_cfg cfg{cut, n_micro};
  if (cu_full > 0) {
    split(cu_full);
    if (cu_slide != cu_full) split(cu_slide);
    if (!rc) {
      if (pools.size() == 2) rc = spa_pipeline_create(t.ctx, t.m, &cfg, pools[0], pools[1], &pipe);
      else rc = spa_pipeline_create_kinds(t.ctx, t.m, &cfg, pools[0], pools[1], pools[2], pools[3], &pipe);
    }
  } else {
    rc = spa_pipeline_create(t.ctx, t.m, &cfg, nullptr, nullptr, &pipe);
  }
  std::vector<double> v;
  for (int i = 0; !rc && i < t.sp->warmup + t.sp->reps; ++i) {
    hipError_t e = hipEventRecord(t.e0, t.st);
    if (e == hipSuccess) {
      rc = spa_pipeline_run(pipe, t.layers, t.b, t.ws, t.ws_bytes, t.st);
      if (!rc) e = hipEventRecord(t.e1, t.st);
      if (!rc && e == hipSuccess) e = hipEventSynchronize(t.e1);
    }
    if (!rc && e != hipSuccess) rc = hip_fail(e, "tuner timing");
    float f = 0.f;
    if (!rc && i >= t.sp->warmup) {
      e = hipEventElapsedTime(&f, t.e0, t.e1);
      if (e != hipSuccess) rc = hip_fail(e, "tuner timing");
      v.push_back(f);
    }
  }
  if (pipe) spa_pipeline_destroy(pipe);
  for (spa_pool* q : pools) spa_pool_destroy(q);
  if (rc) return rc;
  std::sort(v.begin(), v.end());
  *ms = v[v.size() / 2];
  t.points.push_back(spa_tune_point{cu_full > 0 ? cut : -1, n_micro, cu_full, cu_slide, *ms});
  return SPA_OK;
}

// Algorithm 2 objective: the split of one layer kind, the other held fixed
double refine_objective(const int32_t* p, int32_t, void* user) {
  TuneCtx& t = *static_cast<TuneCtx*>(user);
  if (t.err) return 1e30;
  double ms = 0.0;
  const int full = t.refine_kind == SPA_FULL ? p[0] : t.fixed_full;
  const int slide = t.refine_kind == SPA_FULL ? (t.per_kind ? t.fixed_slide : p[0]) : p[0];
  spa_status rc = measure(t, t.cut, t.n_micro, full, t.per_kind ? slide : full, &ms);
  if (rc) {
    t.err = rc;
    return 1e30;
  }
  return ms;
}

}  // namespace

extern "C" spa_status spa_pipeline_tune(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* layers,
                                        const spa_batch* b, void* ws, size_t ws_bytes, const spa_tune_space* sp,
                                        spa_tune_point* best_out, spa_tune_point* points_out, int32_t max_points,
                                        int32_t* n_points, void* stream) {
  if (!ctx || !m || !layers || !b || !ws || !sp || !best_out) return fail(SPA_EINVAL, "bad argument");
  const int nx = ctx->n_xcd;
  if (sp->n_cuts < 1 || sp->n_cuts > 3 || sp->n_micros < 1 || sp->n_micros > 4) return fail(SPA_EINVAL, "bad space");
  if (sp->cu_step < nx || sp->cu_step % nx || sp->cu_min < nx || sp->cu_min % nx || sp->reps < 1 || sp->warmup < 0)
    return fail(SPA_EINVAL, "cu_step and cu_min must be positive multiples of the XCD count; reps >= 1");
  for (int i = 0; i < sp->n_cuts; ++i)
    if (sp->cuts[i] < 0 || sp->cuts[i] > 2) return fail(SPA_EINVAL, "cut must be 0, 1 or 2");
  for (int i = 0; i < sp->n_micros; ++i)
    if (sp->micros[i] < 1 || b->batch % sp->micros[i]) return fail(SPA_EINVAL, "each microbatch count must divide the batch");
  TuneCtx t{ctx, m, layers, b, ws, ws_bytes, sp, (hipStream_t)stream, nullptr, nullptr};
  SPA_HIP(hipEventCreate(&t.e0));
  hipError_t he = hipEventCreate(&t.e1);
  if (he != hipSuccess) {
    (void)hipEventDestroy(t.e0);
    return hip_fail(he, "hipEventCreate");
  }
  spa_status rc = SPA_OK;
  spa_tune_point best{0, 0, 0, 0, 1e30};
  t.per_kind = sp->per_kind != 0;
  for (int mi = 0; !rc && mi < sp->n_micros; ++mi) {
    double ms;
    rc = measure(t, 0, sp->micros[mi], 0, 0, &ms);   // temporal reference
    for (int ci = 0; !rc && ci < sp->n_cuts; ++ci) {
      const bool pk = t.per_kind && sp->cuts[ci] != 2;   // the Macro cut has one split
      for (int cf = sp->cu_min; !rc && cf <= ctx->n_cus - sp->cu_min; cf += sp->cu_step)
        for (int cs = pk ? sp->cu_min : cf; !rc && cs <= (pk ? ctx->n_cus - sp->cu_min : cf); cs += sp->cu_step) {
          rc = measure(t, sp->cuts[ci], sp->micros[mi], cf, cs, &ms);
          if (!rc && ms < best.ms) best = spa_tune_point{sp->cuts[ci], sp->micros[mi], cf, cs, ms};
        }
    }
  }
  if (!rc && sp->refine && best.cu_a > 0) {
    t.cut = best.cut;
    t.n_micro = best.n_micro;
    for (int kind : {SPA_FULL, SPA_SLIDING}) {   // one line search per layer kind (one without per_kind)
      if ((!t.per_kind || best.cut == 2) && kind == SPA_SLIDING) break;
      t.refine_kind = kind;
      t.fixed_full = best.cu_a;
      t.fixed_slide = best.cu_a_sliding;
      const int start = kind == SPA_FULL ? best.cu_a : best.cu_a_sliding;
      int32_t alloc[2] = {start, ctx->n_cus - start};
      double v = 0.0;
      int32_t evals = 0;
      rc = spa_refine_allocation(2, ctx->n_cus, nx, sp->cu_min, alloc, refine_objective, &t, 0, &v, &evals);
      if (!rc) rc = t.err;
      if (rc) break;
      if (v < best.ms) {
        if (kind == SPA_FULL) {
          best.cu_a = alloc[0];
          if (!t.per_kind || best.cut == 2) best.cu_a_sliding = alloc[0];
        } else {
          best.cu_a_sliding = alloc[0];
        }
        best.ms = v;
      }
    }
  }
  (void)hipEventDestroy(t.e0);
  (void)hipEventDestroy(t.e1);
  if (rc) return rc;
  *best_out = best;
  if (n_points) *n_points = (int32_t)t.points.size();
  if (points_out)
    for (size_t i = 0; i < t.points.size() && (int)i < max_points; ++i) points_out[i] = t.points[i];
  return SPA_OK;
}
