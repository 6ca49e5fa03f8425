/*
 * spa.h - C ABI of the MI355X (gfx950) spatially pipelined MoE decode layer.
 *
 * The library runs one GPT-OSS-style MoE transformer decode layer - the
 * operator chain drawn in Figure 3 of "SubGPU Pipelining: Intra-GPU
 * Fine-Grained Spatial Parallelism for LLM Inference" (Andoorveedu et al.,
 * arXiv:2611.14904): RMSNorm, Q/KV projection, attention, output projection,
 * Add+Norm, router gating, top-k dispatch, expert up, SwiGLU, expert down,
 * combine - and repeats it over layers that alternate sliding-window and full
 * attention (its section 5.1). It executes a decode iteration either
 * temporally (every kernel on all CUs, section 5.1 "Temporal") or as the
 * paper's two-stage spatial pipeline (sections 3.1-3.2): the layer is cut
 * into two contiguous segments bound to disjoint CU pools, and microbatches
 * stream through them with event-ordered hand-offs.
 *
 * Conventions
 *   - Every tensor argument is a device pointer to caller-owned memory
 *     (allocated by the caller, e.g. with PyTorch); the library never frees
 *     it. The library owns only the objects it creates: contexts, CU pools
 *     (with their streams) and pipelines.
 *   - Compute calls are asynchronous: they enqueue work on the given HIP
 *     stream (NULL = the null stream) and return. Device faults surface at
 *     the caller's next synchronisation.
 *   - Errors are status codes (spa_status < 0). Arguments are validated on
 *     the host before anything is launched; on error nothing is enqueued and
 *     spa_last_error() describes the problem (thread-local string, valid
 *     until the next call on the same thread).
 *   - Data-dependent errors found on the device (a KV length beyond its
 *     cache capacity) set bits in the workspace error word; read them with
 *     spa_workspace_errors().
 *   - Results are deterministic: every reduction runs in a fixed order, and
 *     launch shapes depend only on tensor shapes, so the spatial pipeline and
 *     the temporal schedule with the same microbatch count give identical
 *     bits.
 *   - Objects are not thread-safe; use one per thread or serialise.
 *
 * Weight layout. Every projection weight is a stack of matrices W[N][K]
 * (N output rows, K inputs) stored in the panel layout that
 * spa_pack_weights() produces from row-major matrices: rows are grouped in
 * panels of 16 (the last one zero-padded) and a panel is stored k-step by
 * k-step, where a k-step is 64 bytes of a row (32 bf16, 16 fp32 or 64 E4M3
 * values); byte b of row n, k-step t of matrix i sits at
 *   ((i * ceil(N/16) + n/16) * (K*esz/64) + t) * 1024 + (n%16) * 64 + b.
 * One k-step of 16 rows is then 1 KB of contiguous memory. As matrices:
 *   wqkv      [(Hq + 2 Hkv) D][H]    rows: q heads, then k heads, then v heads.
 *   wo        [H][Hq D]
 *   wr        [E][H] fp32 (router)
 *   wgu       [E_res][2I][H]  rows 0..I-1 gate, I..2I-1 up (per expert).
 *   wd        [E_res][H][I]
 *   wgu_scale [E_res][2I], wd_scale [E_res][H] fp32 (E4M3 experts only,
 *             plain arrays): dequantised weight = code value * scale of its row.
 *
 * Other tensors (row-major; all offsets in elements)
 *   x         [B][H] fp32 residual stream, updated in place by a layer.
 *   sinks     [Hq] fp32 attention sink logits; gamma1, gamma2 [H] fp32.
 *   KV cache, per layer, D = 64, dtype kv_dtype:
 *     full layers (packed): the region of (sequence s, KV head g) starts at
 *       (kv_off[s] * Hkv + g * kv_cap[s]) * D and holds kv_cap[s] positions
 *       (kv_cap a multiple of 32, kv_len[s] <= kv_cap[s]; regions of
 *       different sequences must not overlap);
 *     sliding layers (ring): region (s * Hkv + g) * W * D holds W slots,
 *       position p in slot p % W (W a multiple of 32);
 *     slots form 32-slot blocks of 32*D elements. K of slot t, dim d at
 *     region + (t/32)*32*D + (d/c)*32*c + (t%32)*c + d%c, c = 64 bytes /
 *     element size (column groups of 64 bytes, slot-major inside a group);
 *     V at region + (t/32)*32*D + d*32 + vslot(t%32), vslot(p) =
 *     8*((p%16)/4) + 4*(p/16) + p%4 (d-major). Use spa_kv_io instead of
 *     computing offsets.
 *   A decode step of sequence s attends positions [0, L) (full) or
 *   [max(0, L-W), L) (sliding), L = kv_len[s], and writes its own K/V at L-1.
 */
#ifndef SPA_H
#define SPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int spa_status;
#define SPA_OK 0
#define SPA_EINVAL (-1)        /* bad argument (shape, pointer, alignment, config) */
#define SPA_EHIP (-2)          /* a HIP runtime call failed */
#define SPA_EWORKSPACE (-3)    /* workspace smaller than spa_workspace_query() */
#define SPA_EUNSUPPORTED (-4)  /* valid but not implemented (shape / dtype combination) */
#define SPA_EMASK (-5)         /* CU mask empty, overlapping, or not honoured by the hardware */

typedef enum { SPA_F32 = 0, SPA_BF16 = 1, SPA_E4M3 = 2 } spa_dtype;
typedef enum { SPA_SLIDING = 0, SPA_FULL = 1 } spa_layer_kind;

/* Model shapes. Constraints: head_dim == 64; Hq % Hkv == 0, Hq/Hkv <= 16;
 * H % 64 == 0; inter % 32 == 0; window % 32 == 0; H, inter, Hq*D multiples
 * of the weight k-step (32 bf16 / 16 fp32 / 64 e4m3 elements);
 * E <= 256; 1 <= top_k <= min(E, 8); 1 <= n_resident <= min(E, 128).
 * dense_dtype: F32 or BF16 (wqkv, wo); expert_dtype: F32, BF16 or E4M3;
 * kv_dtype: F32 or BF16 and equal to dense_dtype. */
typedef struct spa_model_desc {
  int32_t hidden;        /* H */
  int32_t n_q_heads;     /* Hq */
  int32_t n_kv_heads;    /* Hkv */
  int32_t head_dim;      /* D */
  int32_t n_experts;     /* E: router width */
  int32_t n_resident;    /* E_res: experts held here; router pick t runs expert t % E_res */
  int32_t top_k;         /* k */
  int32_t inter;         /* I: expert intermediate width */
  int32_t window;        /* W: sliding-window length */
  int32_t n_layers;
  float eps;             /* RMSNorm epsilon */
  int32_t dense_dtype;
  int32_t expert_dtype;
  int32_t kv_dtype;
  /* Virtual communication endpoints of one rank of a multi-GPU deployment
   * (the single-GPU emulation of section 5.3.1 of the SubGPU Pipelining
   * paper): with comm_gbps > 0, every layer also runs the attention
   * all-reduce after the output projection, the MoE dispatch after the
   * router and the MoE combine after the expert down projection, each as a
   * spa_virtual_comm() launch on its stage's stream whose payload is the
   * tensor that collective would carry (B x H dense_dtype values for the
   * all-reduce, B*k x H expert-input values (+ E4M3 row scales) for
   * dispatch, B*k x H dense_dtype values for combine; B = tokens of the
   * call). Results do not change; only time does. comm_gbps = 0 (the
   * zero-initialised default) leaves them out. 0 <= comm_latency_us <= 1000,
   * 0 <= comm_gbps <= 100000. */
  float comm_latency_us;
  float comm_gbps;
  /* Figure 3 "RoPE": with rope_theta > 0, q and the new k are turned at the
   * decoded position p = L-1 before they are stored (q as the attention
   * input, k into the cache), pair by pair: (v[2i], v[2i+1]) of a head by
   * the angle p * rope_theta^(-2i/D) (RoFormer's rotary embedding; cached
   * keys are taken as already rotated at their own positions). 0 (the
   * zero-initialised default) leaves it out. Finite, >= 0. */
  float rope_theta;
} spa_model_desc;

/* One layer's parameters and KV cache (device pointers). */
typedef struct spa_layer {
  int32_t kind;          /* spa_layer_kind */
  const void* wqkv;
  const void* wo;
  const float* wr;
  const void* wgu;
  const void* wd;
  const float* wgu_scale;   /* E4M3 experts only, else NULL */
  const float* wd_scale;
  const float* gamma1;
  const float* gamma2;
  const float* sinks;
  void* k_cache;
  void* v_cache;
} spa_layer;

/* The decode batch: B sequences, one decoded token each. */
typedef struct spa_batch {
  int32_t batch;              /* B */
  int32_t max_kv_len;         /* host upper bound of kv_len[] (sizes the attention grid) */
  const int32_t* kv_len;      /* device [B]: L (positions incl. the decoded token) */
  const int64_t* kv_off;      /* device [B]: full-layer region start, in positions */
  const int32_t* kv_cap;      /* device [B]: full-layer region capacity (multiple of 32) */
  float* x;                   /* device [B][H] fp32, in/out */
  int32_t* topk_out;          /* optional device [n_layers][B][k]: router picks per layer */
} spa_batch;

/* Router / dispatch buffers of B tokens (device). */
typedef struct spa_route_bufs {
  int32_t* topk_idx;   /* [B][k] router picks 0..E-1, by logit descending, ties to lower index */
  float* topk_w;       /* [B][k] softmax over the k picked logits */
  int32_t* offsets;    /* [E_res + 1] exclusive prefix sum of rows per resident expert */
  int32_t* row_tok;    /* [B*k] dispatch row -> token */
  int32_t* row_slot;   /* [B*k] dispatch row -> pick index */
  int32_t* inv;        /* [B][k] (token, pick) -> dispatch row */
} spa_route_bufs;

typedef struct spa_ctx spa_ctx;
typedef struct spa_pool spa_pool;
typedef struct spa_pipeline spa_pipeline;

/* ---------------------------------------------------------------- context */
spa_status spa_init(int hip_device, spa_ctx** out);
spa_status spa_shutdown(spa_ctx* ctx);
const char* spa_last_error(void);
/* number of CUs of the device (hipDeviceProp_t::multiProcessorCount) */
spa_status spa_device_cus(spa_ctx* ctx, int32_t* n_cus);

/* -------------------------------------------------------------- workspace */
/* Bytes of workspace a call with these shapes needs: n_micro microbatches of
 * batch/n_micro tokens each (n_micro = 1 for the single-op calls). A
 * workspace serves one call at a time: calls that share one must be ordered
 * (one stream, or events), since its header holds the error word and the
 * launch counters (routing arrivals, MoE-head hand-offs) that every call
 * clears and uses. */
spa_status spa_workspace_query(const spa_model_desc* m, int32_t batch, int32_t max_kv_len, int32_t n_micro,
                               size_t* bytes);
/* Prepare a fresh workspace (clears its counters); enqueued on `stream`. */
spa_status spa_workspace_init(spa_ctx* ctx, const spa_model_desc* m, int32_t batch, int32_t max_kv_len,
                              int32_t n_micro, void* ws, size_t ws_bytes, void* stream);
/* Device error bits found so far (1: a kv_len outside its cache; 2: a
 * hand-off inside the one-launch MoE head did not complete within its
 * polling bound, so that launch's results are invalid); synchronises `stream`. */
spa_status spa_workspace_errors(spa_ctx* ctx, const void* ws, size_t ws_bytes, void* stream, int32_t* bits);

/* -------------------------------------------------------------- KV cache */
/* Write (write = 1) or read (write = 0) n cache rows: row r is position pos[r]
 * of sequence seq[r], all KV heads: rows [n][Hkv][D] in kv_dtype. seq/pos are
 * device arrays. kind selects the layer layout (spa_layer_kind). */
spa_status spa_kv_io(spa_ctx* ctx, const spa_model_desc* m, int32_t kind, void* k_cache, void* v_cache,
                     const spa_batch* b, const int32_t* seq, const int32_t* pos, int32_t n, void* k_rows,
                     void* v_rows, int32_t write, void* stream);

/* Bytes of n_mats packed N x K matrices (the panel layout above): n_mats *
 * ceil(N/16)*16 * K * element size. 0 if the shape is not packable (K *
 * element size must be a multiple of 64 bytes). */
size_t spa_packed_bytes(int32_t dtype, int32_t n_mats, int32_t n_rows, int32_t k);

/* Pack n_mats row-major matrices src [n_mats][n_rows][k] (dtype) into the
 * panel layout at dst (spa_packed_bytes() bytes, caller-owned, must not
 * overlap src). Both pointers 16-byte aligned device memory. Asynchronous
 * on `stream`. SPA_EINVAL for a bad dtype, shape, pointer or overlap. */
spa_status spa_pack_weights(spa_ctx* ctx, int32_t dtype, int32_t n_mats, int32_t n_rows, int32_t k, const void* src,
                            void* dst, void* stream);

/* -------------------------------------------------------- single operators
 * Each acts on tokens [tok0, tok0 + n_tok) of the batch and uses `ws`
 * (>= spa_workspace_query(m, n_tok, max_kv_len, 1) bytes). */

/* RMSNorm (Figure 3 "RMSNorm"): xn = x * gamma / sqrt(mean(x^2) + eps) per
 * row of x [n_tok][H] fp32; xn_out [n_tok][H] in dense_dtype (the
 * projection input). */
spa_status spa_rms_norm(spa_ctx* ctx, const spa_model_desc* m, const float* x, const float* gamma, int32_t n_tok,
                        void* xn_out, void* stream);

/* Figure 3 "Q proj, KV proj" (+ "RoPE" when the model's rope_theta > 0):
 * [q | k | v] = xn Wqkv^T from the normalised rows xn [n_tok][H]
 * (dense_dtype); q -> q_out [n_tok][Hq*D] (kv_dtype), k and v -> the layer's
 * cache at position kv_len[s] - 1 of sequence s = tok0 + row. */
spa_status spa_qkv_append(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b,
                          int32_t tok0, int32_t n_tok, const void* xn, void* q_out, void* ws, size_t ws_bytes,
                          void* stream);

/* Figure 3 "FMHA" (section 5.1: sliding or full): grouped-query decode
 * attention with sinks over the cached window; q [n_tok][Hq*D] and o_out
 * [n_tok][Hq*D] in kv_dtype. Split-KV, partial softmax states merged with the
 * sink in window order. Full layers of up to 1024 tokens: the call's windows,
 * laid end to end as 32-position blocks, are cut into 2 x (device CUs) equal
 * ranges, so a window may be cut anywhere and a token's last bits depend on
 * the other tokens' lengths in the call (never on the CU pool). Other calls:
 * a window is cut into equal chunks of at most 4096 .. 512 positions (the
 * largest cap that still gives two workgroups per CU at the batch's longest
 * sequence). */
spa_status spa_decode_attn(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b,
                           int32_t tok0, int32_t n_tok, const void* q, void* o_out, void* ws, size_t ws_bytes,
                           void* stream);

/* spa_decode_attn for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid
 * allocation): the same operator, kernels and results, with no workspace.
 * Its scratch (the softmax partials of the pieces) lives in a fixed array
 * of the library, one per GPU, held until the process ends: at most 24 MiB of
 * partials. A full layer of up to 1024 tokens needs
 * (2 * CUs + n_tok * Hkv) * (Hq/Hkv) * (D + 2) * 4 + n_tok * Hkv * 8 bytes
 * (18.4 MB at 1024 tokens on 256 CUs, 8 KV heads of 8 query heads); other
 * calls need
 * n_tok * Hkv * chunks * (Hq/Hkv) * (D + 2) * 4 bytes, where
 * chunks = ceil(max_kv_len / chunk) for full layers (the chunk is 4096 ..
 * 512 positions, chosen from the shapes as in spa_decode_attn) and
 * ceil(window / 512) for sliding layers. A call that needs more returns
 * SPA_EWORKSPACE and enqueues nothing. The call allocates nothing.
 * err_out: optional device int32, zeroed by the caller; bit 0 is set when a
 * kv_len lies outside its cache (those rows are then left unwritten). With
 * err_out NULL the bit goes to the array's own word, which the caller
 * cannot read. Every call on one GPU shares that GPU's array and the array
 * keeps the last call's contents: calls that overlap in time on one GPU
 * (different streams, or different host threads) race and must be
 * serialised by the caller. */
spa_status spa_decode_attn_noalloc(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const spa_batch* b,
                                   int32_t tok0, int32_t n_tok, const void* q, void* o_out, int32_t* err_out,
                                   void* stream);

/* Figure 3 "Output proj, Add+Norm": h = x + o Wo^T (h_out [n_tok][H] fp32)
 * and hn = RMSNorm(h) gamma2 (hn_out [n_tok][H] fp32). */
spa_status spa_out_proj(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* x, const void* o,
                        int32_t n_tok, float* h_out, float* hn_out, void* ws, size_t ws_bytes, void* stream);

/* Figure 3 "Router gating, TopK dispatch": logits = hn Wr^T (fp32, hn
 * [n_tok][H] fp32); top-k + softmax over the picks; permutation of (token,
 * pick) rows grouped by resident expert (pick t -> expert t % E_res),
 * (token, pick) ascending inside an expert. */
spa_status spa_moe_route(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* hn, int32_t n_tok,
                         float* logits_out, const spa_route_bufs* r, int32_t* topk_rec, void* ws, size_t ws_bytes,
                         void* stream);

/* Figure 3 "Expert up (BMM), SwiGLU, Expert down": for each dispatch row,
 * with x = hn of its token in the expert input format (bf16, or per-row
 * power-of-two-scaled E4M3): z = silu(x Wg^T) * (x Wu^T), y = z Wd^T
 * (y_out [n_tok*k][H] fp32, dispatch row order). */
spa_status spa_moe_expert(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, const float* hn, int32_t n_tok,
                          const spa_route_bufs* r, float* y_out, void* ws, size_t ws_bytes, void* stream);

/* Figure 3 "Combine": x_out = h + sum over picks (in pick order) of w * y;
 * when gamma_next is given, also xn_out = RMSNorm(x_out) gamma_next (the next
 * layer's projection input, dense_dtype). */
spa_status spa_moe_combine(spa_ctx* ctx, const spa_model_desc* m, const float* h, const float* y,
                           const spa_route_bufs* r, int32_t n_tok, float* x_out, const float* gamma_next, void* xn_out,
                           void* stream);

/* A virtual communication endpoint (section 5.3.1 of the paper: a collective
 * of a multi-GPU rank replaced by a kernel that does the endpoint's local
 * work and lasts the modelled time). Copies `bytes` bytes from src to dst
 * (device memory, 16-byte aligned, not overlapping; the endpoint's read of
 * the send buffer and write of the receive buffer) and keeps the launch
 * running until latency_us + bytes / (gbps * 1e3) microseconds after each
 * workgroup started, on the device wall clock. bytes <= 2^32; the modelled
 * time must stay below 100 ms; SPA_EINVAL otherwise. bytes = 0 is a pure
 * delay (src, dst may be NULL). */
spa_status spa_virtual_comm(spa_ctx* ctx, const void* src, void* dst, size_t bytes, float latency_us, float gbps,
                            void* stream);

/* One whole layer, temporal, on tokens [tok0, tok0 + n_tok): updates x in
 * place, appends K/V, optionally records the router picks. */
spa_status spa_layer_forward(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* l, int32_t layer_index,
                             const spa_batch* b, int32_t tok0, int32_t n_tok, void* ws, size_t ws_bytes,
                             void* stream);

/* ------------------------------------------------------ decode iteration */
/* Temporal execution (section 5.1 "Temporal"): the n_layers layers in order,
 * each kernel on the whole device, the batch split into n_micro equal
 * microbatches processed one after another on `stream`. */
spa_status spa_temporal_run(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* layers, const spa_batch* b,
                            int32_t n_micro, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------- CU pools
 * The HIP analogue of an SM partition (section 2.4 of the paper): a pool is
 * a set of CUs with its own stream(s) whose kernels may only run on those
 * CUs (hipExtStreamCreateWithCUMask). Masks are given in the runtime's CU
 * mask bit order (bit i of word i/32). */
spa_status spa_pool_create_mask(spa_ctx* ctx, const uint32_t* cu_mask, int32_t n_words, spa_pool** out);
/* A pool of n_cus CUs spread evenly over the XCDs; `first` selects which CUs
 * of each XCD (pools built with disjoint [first, first + n_cus/n_xcd) ranges
 * are disjoint). n_cus must be a multiple of the XCD count. */
spa_status spa_pool_create_split(spa_ctx* ctx, int32_t first_per_xcd, int32_t n_cus, spa_pool** out);
spa_status spa_pool_mask(spa_pool* p, uint32_t* mask_out, int32_t n_words);
spa_status spa_pool_stream(spa_pool* p, void** hip_stream);
/* Placement probe: launch many short workgroups on the pool's stream and
 * report the distinct hardware CUs (XCC, SE, SH, CU ids packed as
 * xcc << 16 | se << 8 | sh << 4 | cu) they ran on, up to max_ids entries. */
spa_status spa_pool_probe(spa_pool* p, int32_t n_blocks, uint32_t* ids_out, int32_t max_ids, int32_t* n_ids);
/* Placement check of a pool (the blog on the paper warns that a partition
 * handle that is not applied silently runs the work on the whole GPU): runs
 * the probe with 64 workgroups per CU of the mask and compares the CUs they
 * landed on with the mask. SPA_OK when they fit it - no more distinct CUs
 * than the mask holds, on as many XCDs, and on no XCD more CUs than the mask
 * gives that XCD (the counts are compared as sorted lists, since the
 * hardware's XCD labels need not follow the mask's numbering); SPA_EMASK
 * otherwise, with the counts in spa_last_error(). observed_out (optional):
 * the distinct CUs seen. Synchronises the pool's stream. */
spa_status spa_pool_verify(spa_pool* p, int32_t* observed_out);
spa_status spa_pool_destroy(spa_pool* p);

/* Read-bandwidth probe (the empirical HBM bandwidth-versus-concurrency curve
 * that section 4.3 of the paper lists among its calibration inputs): n_wgs
 * workgroups of 256 threads each stream their share of `bytes` bytes of src
 * once (non-temporal 16-byte loads, 8 in flight per lane) on `stream`; on a
 * pool's stream this is the rate that pool can pull. src: device memory,
 * 16-byte aligned; bytes a non-zero multiple of n_wgs * 1024. One warm-up
 * launch, then `reps` launches between two events; *ms = mean launch time.
 * Synchronises the stream. The rate is bytes / ms. */
spa_status spa_hbm_probe(spa_ctx* ctx, const void* src, size_t bytes, int32_t n_wgs, int32_t reps, void* stream,
                         double* ms);

/* --------------------------------------------------------- the pipeline
 * theta = (D = 2 stages, w, cut, CU split, microbatch count) of section
 * 3.1. Cuts 0 and 1 (w = 0): stage A holds the segment up to the cut, stage
 * B the rest:
 *   cut 0: A = Norm+QKV, attention, output projection (+ residual) | B = router ... combine
 *   cut 1: A = Norm+QKV, attention, output projection, router       | B = experts, combine
 * Cut 2, the "Macro" design of section 5.3.2 (w = 1 over a two-layer
 * period): stage A runs only the attention of full layers; stage B runs
 * everything else - per full layer F and microbatch mu, the rest of the
 * previous full layer (output projection .. combine), the sliding layers
 * in between, and F's Norm+QKV - so B(F, mu) -> A(F, mu) -> B(next, mu).
 * Sliding-layer pools are not used by cut 2.
 * Microbatch mu is the contiguous token slice [mu*B/m, (mu+1)*B/m). Tasks are
 * dispatched region-major, then microbatch (a topological order of the data
 * edges, section 3.2); each stage runs its tasks in that order (stage FIFO);
 * A(l, mu) waits for B(l-1, mu) and B(l, mu) for A(l, mu): the finishing
 * stream writes a per-microbatch counter in device memory and the other
 * stream waits for it (stream value write/wait; events where the runtime
 * lacks them, or when `handoff` asks for them). */
typedef struct spa_pipeline_cfg {
  int32_t cut;        /* 0, 1 or 2 (Macro) */
  int32_t n_micro;    /* m, divides the batch */
  /* Stage hand-off mechanism. 0 (the zero-initialised default): stream value
   * write/wait on device counters where the runtime supports them. 1:
   * event record/wait always. The runtime executes a value wait as a small
   * kernel that polls memory; a tool that runs one dispatch at a time (a
   * per-dispatch hardware-counter collection) can then leave that poller
   * waiting for a write whose dispatch it holds back. Event waits are
   * resolved by the command processor and dispatch nothing, so use 1 under
   * such tools. Results are identical either way. */
  int32_t handoff;
  /* 1: temporal pipelines (no pools) capture an iteration's launches into a
   * HIP graph on its own stream the first time and replay it while the
   * run's arguments (layers, batch, workspace, kernel timer) are unchanged,
   * capturing again when they change; the graph replaces about 360 kernel
   * launches per 36-layer iteration with one. Same kernels, same results
   * (for callers that must submit whole iterations; on the 36-layer batch-64
   * workload it measured 6.79 ms per iteration against 6.38 ms launched
   * directly).
   * Spatial pipelines refuse it (SPA_EUNSUPPORTED): graph kernel nodes do
   * not keep a stream's CU mask. 0 (default): direct launches. */
  int32_t graph;
  /* 1: the MoE head - output projection finish, router GEMV, top-k, the
   * dispatch permutation and the gather of the expert rows - as one
   * persistent launch: up to 64 workgroups (at most one per CU of the
   * stream's pool, so all are resident) run the four steps with device
   * hand-offs between them (agent-scope release, an arrival counter,
   * bounded polling, agent-scope acquire) instead of four dependent
   * launches (the "persistent kernels" of section 6.1 of the paper). Same
   * arithmetic as the separate kernels, same bits. Used wherever the output
   * projection and the router share a stream (temporal schedules, cuts 1
   * and 2), every stage has one pool, the virtual communication endpoints
   * are off and the shapes fit its instances; elsewhere the separate
   * launches run. On the 36-layer batch-64 workload the one launch took
   * 36 us against 25 us for the four it replaces. 0 (default): the separate
   * launches. */
  int32_t head;
} spa_pipeline_cfg;

spa_status spa_pipeline_create(spa_ctx* ctx, const spa_model_desc* m, const spa_pipeline_cfg* cfg, spa_pool* stage_a,
                               spa_pool* stage_b, spa_pipeline** out);
/* The same pipeline with a CU split per layer kind: full layers run stage A
 * on a_full and stage B on b_full, sliding layers on a_sliding / b_sliding
 * (full layers are attention-heavy, sliding layers MoE-heavy). The pools of
 * one kind must be disjoint; pools of different kinds may overlap (tasks of
 * adjacent layers then share CUs). spa_pipeline_create(a, b) is the case
 * a_full = a_sliding = a, b_full = b_sliding = b. */
spa_status spa_pipeline_create_kinds(spa_ctx* ctx, const spa_model_desc* m, const spa_pipeline_cfg* cfg,
                                     spa_pool* a_full, spa_pool* b_full, spa_pool* a_sliding, spa_pool* b_sliding,
                                     spa_pipeline** out);
/* Run one decode iteration; joins `caller_stream` at both ends (the pipeline
 * starts after work already queued there, and work queued there afterwards
 * starts after the iteration). */
spa_status spa_pipeline_run(spa_pipeline* p, const spa_layer* layers, const spa_batch* b, void* ws, size_t ws_bytes,
                            void* caller_stream);
/* Per-kernel timing of every launch of kernel class `cls` (0 = full-layer
 * attention, 1 = sliding attention, 2 = QKV, 3 = output projection, 4 =
 * router, 5 = expert gate/up, 6 = expert down, 7 = combine, 8 = virtual
 * communication endpoints).
 * enable = 0: off.
 * enable = 1: for the attention classes the kernel itself records its span on
 *   the device wall clock (start of the first dispatched workgroup to the
 *   latest workgroup end; one atomic per workgroup, no extra packets in
 *   the queue); the other
 *   classes fall back to mode 2. Spans of up to 8192 launches are kept
 *   between two harvests (spa_pipeline_timing or a new enable); later
 *   launches run untimed.
 * enable = 2: HIP events recorded around each launch on its stream. Their
 *   interval also holds the start marker's dispatch latency, and the
 *   markers delay the launch they bracket.
 * spa_pipeline_timing synchronises the device and returns the mean duration
 * (ms) over the launches timed since enabling, and their count. SPA_EINVAL
 * for a bad class or mode. */
spa_status spa_pipeline_time_kernel(spa_pipeline* p, int32_t cls, int32_t enable);
spa_status spa_pipeline_timing(spa_pipeline* p, double* mean_ms, int32_t* count);
spa_status spa_pipeline_destroy(spa_pipeline* p);

/* ---------------------------------------------------------------- tuner
 * Section 4 (offline search, online selection): measure the iteration time
 * T(theta) of every point of a small grid - cut x stage A's CU count (per
 * layer kind with per_kind) x microbatch count - on the caller's own layers
 * and batch, then refine the CU split(s) of the best point with Algorithm 2
 * (spa_refine_allocation) using measured times as the objective. Temporal runs (cu_a = 0) of every
 * microbatch count are measured too, for reference. Each point runs
 * `warmup` untimed and `reps` timed iterations, each timed one after the
 * other (the previous one complete); the median is kept.
 * The runs update x and the KV caches like any iteration (restore them if
 * they matter). The workspace must fit every point (the largest of
 * spa_workspace_query() over the microbatch counts). */
typedef struct spa_tune_space {
  int32_t n_cuts;        /* 1 to 3 entries of cuts (each 0, 1 or 2) */
  int32_t cuts[3];
  int32_t n_micros;      /* 1..4 entries of micros, each dividing the batch */
  int32_t micros[4];
  int32_t cu_step;       /* grid spacing of stage A's CU count: a multiple of the XCD count */
  int32_t cu_min;        /* smallest pool, a multiple of the XCD count */
  int32_t warmup;
  int32_t reps;
  int32_t refine;        /* 1: Algorithm 2 on the best grid point's split(s) */
  int32_t per_kind;      /* 1: search stage A's CUs for full and sliding layers separately */
} spa_tune_space;

typedef struct spa_tune_point {
  int32_t cut;           /* -1 for temporal points */
  int32_t n_micro;
  int32_t cu_a;          /* stage A's CUs (full layers); 0 for temporal points */
  int32_t cu_a_sliding;  /* stage A's CUs for sliding layers (= cu_a without per_kind) */
  double ms;             /* median iteration time */
} spa_tune_point;

/* best_out: the fastest spatial point. points_out (optional, max_points
 * entries): every measured point in measurement order; n_points gets the
 * total count (may exceed max_points). */
spa_status spa_pipeline_tune(spa_ctx* ctx, const spa_model_desc* m, const spa_layer* layers, const spa_batch* b,
                             void* ws, size_t ws_bytes, const spa_tune_space* space, spa_tune_point* best_out,
                             spa_tune_point* points_out, int32_t max_points, int32_t* n_points, void* stream);

/* ------------------------------------------------- schedule model (host)
 * Equations 1, 4 and 5 of the paper: binding of segment k (1-based) of K
 * with boundary reuse w, and the max-plus makespan of n_regions x n_micro x
 * K segment tasks with durations tau[(l * n_micro + mu) * K + (k - 1)] in the
 * region-major dispatch order. */
int32_t spa_sched_binding(int32_t k, int32_t K, int32_t w);
spa_status spa_sched_makespan(int32_t n_regions, int32_t n_micro, int32_t K, int32_t w, const double* tau,
                              double* makespan, double* start_out, double* end_out);
/* Equation 7's counts: contiguous cut-and-binding choices of an n_ops chain
 * for n_stages (K = D and K = D + 1), and ordered full-budget allocations of
 * n_units to n_stages in positive multiples of quantum. */
spa_status spa_sched_counts(int32_t n_ops, int32_t n_stages, int32_t n_units, int32_t quantum, int64_t* cut_choices,
                            int64_t* allocations);

/* Section 4.2, Algorithm 2 (pairwise-line refinement): improve an
 * allocation p[n_stages] (positive multiples of quantum, at least p_min,
 * summing to total) by moving quanta between one donor and one receiver
 * stage per pass. objective(p, user) returns the value to minimise.
 * pass_limit <= 0 means no limit. */
typedef double (*spa_objective_fn)(const int32_t* p, int32_t n_stages, void* user);
spa_status spa_refine_allocation(int32_t n_stages, int32_t total, int32_t quantum, int32_t p_min, int32_t* p,
                                 spa_objective_fn objective, void* user, int32_t pass_limit, double* best,
                                 int32_t* n_evals);

#ifdef __cplusplus
}
#endif

#endif /* SPA_H */
