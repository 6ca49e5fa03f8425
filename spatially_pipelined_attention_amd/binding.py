"""ctypes binding of libspa.so (include/spa.h): same names, argument marshalling only.

Tensors are passed as torch CUDA tensors (their data pointers); streams as
torch streams or raw HIP stream handles. Every function raises SpaError on a
non-zero status. Importing this module needs the built library; it never
falls back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPA_LIBRARY names another build of the same library (a build-time variant
# for a measurement); the default is the in-tree build.
LIB_PATH = os.environ.get("SPA_LIBRARY") or os.path.join(_HERE, "libspa.so")

SPA_OK = 0
SPA_EINVAL = -1
SPA_EHIP = -2
SPA_EWORKSPACE = -3
SPA_EUNSUPPORTED = -4
SPA_EMASK = -5

SPA_F32, SPA_BF16, SPA_E4M3 = 0, 1, 2
SPA_SLIDING, SPA_FULL = 0, 1

KC_ATTN_FULL, KC_ATTN_SLIDING, KC_QKV, KC_OPROJ, KC_ROUTER, KC_GATEUP, KC_DOWN, KC_COMBINE, KC_COMM = range(9)


class SpaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"spa status {status}: {msg}")
        self.status = status


class spa_model_desc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("n_experts", C.c_int32), ("n_resident", C.c_int32),
                ("top_k", C.c_int32), ("inter", C.c_int32), ("window", C.c_int32), ("n_layers", C.c_int32),
                ("eps", C.c_float), ("dense_dtype", C.c_int32), ("expert_dtype", C.c_int32),
                ("kv_dtype", C.c_int32), ("comm_latency_us", C.c_float), ("comm_gbps", C.c_float),
                ("rope_theta", C.c_float)]


class spa_layer(C.Structure):
    _fields_ = [("kind", C.c_int32), ("wqkv", C.c_void_p), ("wo", C.c_void_p), ("wr", C.c_void_p),
                ("wgu", C.c_void_p), ("wd", C.c_void_p), ("wgu_scale", C.c_void_p), ("wd_scale", C.c_void_p),
                ("gamma1", C.c_void_p), ("gamma2", C.c_void_p), ("sinks", C.c_void_p), ("k_cache", C.c_void_p),
                ("v_cache", C.c_void_p)]


class spa_batch(C.Structure):
    _fields_ = [("batch", C.c_int32), ("max_kv_len", C.c_int32), ("kv_len", C.c_void_p), ("kv_off", C.c_void_p),
                ("kv_cap", C.c_void_p), ("x", C.c_void_p), ("topk_out", C.c_void_p)]


class spa_route_bufs(C.Structure):
    _fields_ = [("topk_idx", C.c_void_p), ("topk_w", C.c_void_p), ("offsets", C.c_void_p),
                ("row_tok", C.c_void_p), ("row_slot", C.c_void_p), ("inv", C.c_void_p)]


class spa_pipeline_cfg(C.Structure):
    _fields_ = [("cut", C.c_int32), ("n_micro", C.c_int32), ("handoff", C.c_int32), ("graph", C.c_int32),
                ("head", C.c_int32)]


class spa_tune_space(C.Structure):
    _fields_ = [("n_cuts", C.c_int32), ("cuts", C.c_int32 * 3), ("n_micros", C.c_int32), ("micros", C.c_int32 * 4),
                ("cu_step", C.c_int32), ("cu_min", C.c_int32), ("warmup", C.c_int32), ("reps", C.c_int32),
                ("refine", C.c_int32), ("per_kind", C.c_int32)]


class spa_tune_point(C.Structure):
    _fields_ = [("cut", C.c_int32), ("n_micro", C.c_int32), ("cu_a", C.c_int32), ("cu_a_sliding", C.c_int32),
                ("ms", C.c_double)]


OBJECTIVE_FN = C.CFUNCTYPE(C.c_double, C.POINTER(C.c_int32), C.c_int32, C.c_void_p)

_P = C.c_void_p
_I = C.c_int32
_PROTOS = {
    "spa_init": [C.c_int, C.POINTER(C.c_void_p)],
    "spa_shutdown": [_P],
    "spa_device_cus": [_P, C.POINTER(C.c_int32)],
    "spa_workspace_query": [C.POINTER(spa_model_desc), _I, _I, _I, C.POINTER(C.c_size_t)],
    "spa_workspace_init": [_P, C.POINTER(spa_model_desc), _I, _I, _I, _P, C.c_size_t, _P],
    "spa_workspace_errors": [_P, _P, C.c_size_t, _P, C.POINTER(C.c_int32)],
    "spa_kv_io": [_P, C.POINTER(spa_model_desc), _I, _P, _P, C.POINTER(spa_batch), _P, _P, _I, _P, _P, _I, _P],
    "spa_pack_weights": [_P, _I, _I, _I, _I, _P, _P, _P],
    "spa_rms_norm": [_P, C.POINTER(spa_model_desc), _P, _P, _I, _P, _P],
    "spa_qkv_append": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), C.POINTER(spa_batch), _I, _I, _P, _P,
                       _P, C.c_size_t, _P],
    "spa_decode_attn": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), C.POINTER(spa_batch), _I, _I, _P, _P,
                        _P, C.c_size_t, _P],
    "spa_decode_attn_noalloc": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), C.POINTER(spa_batch), _I, _I,
                                _P, _P, _P, _P],
    "spa_out_proj": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), _P, _P, _I, _P, _P, _P, C.c_size_t, _P],
    "spa_moe_route": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), _P, _I, _P,
                      C.POINTER(spa_route_bufs), _P, _P, C.c_size_t, _P],
    "spa_moe_expert": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), _P, _I, C.POINTER(spa_route_bufs),
                       _P, _P, C.c_size_t, _P],
    "spa_moe_combine": [_P, C.POINTER(spa_model_desc), _P, _P, C.POINTER(spa_route_bufs), _I, _P, _P, _P, _P],
    "spa_virtual_comm": [_P, _P, _P, C.c_size_t, C.c_float, C.c_float, _P],
    "spa_layer_forward": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), _I, C.POINTER(spa_batch), _I, _I, _P,
                          C.c_size_t, _P],
    "spa_temporal_run": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), C.POINTER(spa_batch), _I, _P,
                         C.c_size_t, _P],
    "spa_pool_create_mask": [_P, C.POINTER(C.c_uint32), _I, C.POINTER(C.c_void_p)],
    "spa_pool_create_split": [_P, _I, _I, C.POINTER(C.c_void_p)],
    "spa_pool_mask": [_P, C.POINTER(C.c_uint32), _I],
    "spa_pool_stream": [_P, C.POINTER(C.c_void_p)],
    "spa_pool_probe": [_P, _I, C.POINTER(C.c_uint32), _I, C.POINTER(C.c_int32)],
    "spa_pool_verify": [_P, C.POINTER(C.c_int32)],
    "spa_hbm_probe": [_P, _P, C.c_size_t, _I, _I, _P, C.POINTER(C.c_double)],
    "spa_pool_destroy": [_P],
    "spa_pipeline_create": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_pipeline_cfg), _P, _P,
                            C.POINTER(C.c_void_p)],
    "spa_pipeline_create_kinds": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_pipeline_cfg), _P, _P, _P, _P,
                                  C.POINTER(C.c_void_p)],
    "spa_pipeline_run": [_P, C.POINTER(spa_layer), C.POINTER(spa_batch), _P, C.c_size_t, _P],
    "spa_pipeline_time_kernel": [_P, _I, _I],
    "spa_pipeline_timing": [_P, C.POINTER(C.c_double), C.POINTER(C.c_int32)],
    "spa_pipeline_destroy": [_P],
    "spa_pipeline_tune": [_P, C.POINTER(spa_model_desc), C.POINTER(spa_layer), C.POINTER(spa_batch), _P, C.c_size_t,
                          C.POINTER(spa_tune_space), C.POINTER(spa_tune_point), C.POINTER(spa_tune_point), _I,
                          C.POINTER(C.c_int32), _P],
    "spa_sched_makespan": [_I, _I, _I, _I, C.POINTER(C.c_double), C.POINTER(C.c_double), C.POINTER(C.c_double),
                           C.POINTER(C.c_double)],
    "spa_sched_counts": [_I, _I, _I, _I, C.POINTER(C.c_int64), C.POINTER(C.c_int64)],
    "spa_refine_allocation": [_I, _I, _I, _I, C.POINTER(C.c_int32), OBJECTIVE_FN, _P, _I, C.POINTER(C.c_double),
                              C.POINTER(C.c_int32)],
}

EXPORTED = sorted(list(_PROTOS) + ["spa_last_error", "spa_sched_binding", "spa_packed_bytes"])

_lib = None


def lib():
    """The loaded libspa.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        for name, args in _PROTOS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.spa_last_error.restype = C.c_char_p
        L.spa_last_error.argtypes = []
        L.spa_sched_binding.restype = C.c_int32
        L.spa_sched_binding.argtypes = [_I, _I, _I]
        L.spa_packed_bytes.restype = C.c_size_t
        L.spa_packed_bytes.argtypes = [_I, _I, _I, _I]
        _lib = L
    return _lib


def _check(rc: int):
    if rc != SPA_OK:
        raise SpaError(rc, lib().spa_last_error().decode())


def ptr(t) -> int | None:
    """Device pointer of a torch tensor (None -> NULL)."""
    return None if t is None else t.data_ptr()


def stream_handle(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ----------------------------------------------------------------------- context
def spa_init(device: int = 0) -> int:
    h = C.c_void_p()
    _check(lib().spa_init(device, C.byref(h)))
    return h.value


def spa_shutdown(ctx: int):
    _check(lib().spa_shutdown(ctx))


def spa_last_error() -> str:
    return lib().spa_last_error().decode()


def spa_device_cus(ctx: int) -> int:
    n = C.c_int32()
    _check(lib().spa_device_cus(ctx, C.byref(n)))
    return n.value


def spa_workspace_query(m: spa_model_desc, batch: int, max_kv_len: int, n_micro: int) -> int:
    n = C.c_size_t()
    _check(lib().spa_workspace_query(C.byref(m), batch, max_kv_len, n_micro, C.byref(n)))
    return n.value


def spa_workspace_init(ctx, m, batch, max_kv_len, n_micro, ws, stream=None):
    _check(lib().spa_workspace_init(ctx, C.byref(m), batch, max_kv_len, n_micro, ptr(ws), ws.numel() * ws.element_size(),
                                     stream_handle(stream)))


def spa_workspace_errors(ctx, ws, stream=None) -> int:
    v = C.c_int32()
    _check(lib().spa_workspace_errors(ctx, ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream), C.byref(v)))
    return v.value


def spa_kv_io(ctx, m, kind, k_cache, v_cache, batch: spa_batch | None, seq, pos, n, k_rows, v_rows, write, stream=None):
    _check(lib().spa_kv_io(ctx, C.byref(m), kind, ptr(k_cache), ptr(v_cache), C.byref(batch) if batch else None,
                           ptr(seq), ptr(pos), n, ptr(k_rows), ptr(v_rows), write, stream_handle(stream)))


def spa_packed_bytes(dtype: int, n_mats: int, n_rows: int, k: int) -> int:
    return int(lib().spa_packed_bytes(dtype, n_mats, n_rows, k))


def spa_pack_weights(ctx, dtype: int, n_mats: int, n_rows: int, k: int, src, dst, stream=None):
    _check(lib().spa_pack_weights(ctx, dtype, n_mats, n_rows, k, ptr(src), ptr(dst), stream_handle(stream)))


# ----------------------------------------------------------------------- operators
def _ws(ws):
    return ptr(ws), ws.numel() * ws.element_size()


def spa_rms_norm(ctx, m, x, gamma, n_tok, xn_out, stream=None):
    _check(lib().spa_rms_norm(ctx, C.byref(m), ptr(x), ptr(gamma), n_tok, ptr(xn_out), stream_handle(stream)))


def spa_qkv_append(ctx, m, layer, batch, tok0, n_tok, xn, q_out, ws, stream=None):
    _check(lib().spa_qkv_append(ctx, C.byref(m), C.byref(layer), C.byref(batch), tok0, n_tok, ptr(xn), ptr(q_out),
                                *_ws(ws), stream_handle(stream)))


def spa_decode_attn(ctx, m, layer, batch, tok0, n_tok, q, o_out, ws, stream=None):
    _check(lib().spa_decode_attn(ctx, C.byref(m), C.byref(layer), C.byref(batch), tok0, n_tok, ptr(q), ptr(o_out),
                                 *_ws(ws), stream_handle(stream)))


def spa_decode_attn_noalloc(ctx, m, layer, batch, tok0, n_tok, q, o_out, err_out=None, stream=None):
    _check(lib().spa_decode_attn_noalloc(ctx, C.byref(m), C.byref(layer), C.byref(batch), tok0, n_tok, ptr(q),
                                         ptr(o_out), ptr(err_out) if err_out is not None else None,
                                         stream_handle(stream)))


def spa_out_proj(ctx, m, layer, x, o, n_tok, h_out, hn_out, ws, stream=None):
    _check(lib().spa_out_proj(ctx, C.byref(m), C.byref(layer), ptr(x), ptr(o), n_tok, ptr(h_out), ptr(hn_out),
                              *_ws(ws), stream_handle(stream)))


def spa_moe_route(ctx, m, layer, hn, n_tok, logits_out, route: spa_route_bufs, topk_rec, ws, stream=None):
    _check(lib().spa_moe_route(ctx, C.byref(m), C.byref(layer), ptr(hn), n_tok, ptr(logits_out), C.byref(route),
                               ptr(topk_rec), *_ws(ws), stream_handle(stream)))


def spa_moe_expert(ctx, m, layer, hn, n_tok, route: spa_route_bufs, y_out, ws, stream=None):
    _check(lib().spa_moe_expert(ctx, C.byref(m), C.byref(layer), ptr(hn), n_tok, C.byref(route), ptr(y_out),
                                *_ws(ws), stream_handle(stream)))


def spa_moe_combine(ctx, m, h, y, route: spa_route_bufs, n_tok, x_out, gamma_next=None, xn_out=None, stream=None):
    _check(lib().spa_moe_combine(ctx, C.byref(m), ptr(h), ptr(y), C.byref(route), n_tok, ptr(x_out), ptr(gamma_next),
                                 ptr(xn_out), stream_handle(stream)))


def spa_virtual_comm(ctx, src, dst, nbytes: int, latency_us: float, gbps: float, stream=None):
    _check(lib().spa_virtual_comm(ctx, ptr(src), ptr(dst), nbytes, latency_us, gbps, stream_handle(stream)))


def spa_layer_forward(ctx, m, layer, layer_index, batch, tok0, n_tok, ws, stream=None):
    _check(lib().spa_layer_forward(ctx, C.byref(m), C.byref(layer), layer_index, C.byref(batch), tok0, n_tok, *_ws(ws),
                                   stream_handle(stream)))


def spa_temporal_run(ctx, m, layers, batch, n_micro, ws, stream=None):
    _check(lib().spa_temporal_run(ctx, C.byref(m), layers, C.byref(batch), n_micro, *_ws(ws), stream_handle(stream)))


# ----------------------------------------------------------------------- pools / pipeline
def spa_pool_create_mask(ctx, mask_words) -> int:
    arr = (C.c_uint32 * len(mask_words))(*mask_words)
    h = C.c_void_p()
    _check(lib().spa_pool_create_mask(ctx, arr, len(mask_words), C.byref(h)))
    return h.value


def spa_pool_create_split(ctx, first_per_xcd: int, n_cus: int) -> int:
    h = C.c_void_p()
    _check(lib().spa_pool_create_split(ctx, first_per_xcd, n_cus, C.byref(h)))
    return h.value


def spa_pool_mask(pool, n_words: int = 8):
    arr = (C.c_uint32 * n_words)()
    _check(lib().spa_pool_mask(pool, arr, n_words))
    return list(arr)


def spa_pool_stream(pool) -> int:
    h = C.c_void_p()
    _check(lib().spa_pool_stream(pool, C.byref(h)))
    return h.value


def spa_pool_probe(pool, n_blocks: int, max_ids: int = 1024):
    arr = (C.c_uint32 * max_ids)()
    n = C.c_int32()
    _check(lib().spa_pool_probe(pool, n_blocks, arr, max_ids, C.byref(n)))
    return list(arr[: min(n.value, max_ids)]), n.value


def spa_pool_verify(pool) -> int:
    """Raises SpaError (SPA_EMASK) when the pool's kernels land outside its mask;
    returns the distinct CUs observed."""
    n = C.c_int32()
    _check(lib().spa_pool_verify(pool, C.byref(n)))
    return n.value


def spa_hbm_probe(ctx, src, n_wgs: int, reps: int = 10, stream=None, nbytes: int | None = None) -> float:
    """Mean launch time (ms) of the read probe over src (a torch CUDA tensor)."""
    ms = C.c_double()
    nb = nbytes if nbytes is not None else src.numel() * src.element_size()
    _check(lib().spa_hbm_probe(ctx, ptr(src), nb, n_wgs, reps, stream_handle(stream), C.byref(ms)))
    return ms.value


def spa_pool_destroy(pool):
    _check(lib().spa_pool_destroy(pool))


def spa_pipeline_create(ctx, m, cfg: spa_pipeline_cfg, pool_a, pool_b) -> int:
    h = C.c_void_p()
    _check(lib().spa_pipeline_create(ctx, C.byref(m), C.byref(cfg), pool_a, pool_b, C.byref(h)))
    return h.value


def spa_pipeline_create_kinds(ctx, m, cfg: spa_pipeline_cfg, a_full, b_full, a_sliding, b_sliding) -> int:
    h = C.c_void_p()
    _check(lib().spa_pipeline_create_kinds(ctx, C.byref(m), C.byref(cfg), a_full, b_full, a_sliding, b_sliding,
                                           C.byref(h)))
    return h.value


def spa_pipeline_run(pipe, layers, batch, ws, stream=None):
    _check(lib().spa_pipeline_run(pipe, layers, C.byref(batch), *_ws(ws), stream_handle(stream)))


def spa_pipeline_time_kernel(pipe, cls: int, enable: int):
    """enable: 0 off, 1 device-clock spans (attention; events otherwise), 2 events."""
    _check(lib().spa_pipeline_time_kernel(pipe, cls, int(enable)))


def spa_pipeline_timing(pipe):
    ms = C.c_double()
    n = C.c_int32()
    _check(lib().spa_pipeline_timing(pipe, C.byref(ms), C.byref(n)))
    return ms.value, n.value


def spa_pipeline_destroy(pipe):
    _check(lib().spa_pipeline_destroy(pipe))


def spa_pipeline_tune(ctx, m, layers, batch, ws, space: spa_tune_space, stream=None, max_points: int = 512):
    best = spa_tune_point()
    pts = (spa_tune_point * max_points)()
    n = C.c_int32()
    _check(lib().spa_pipeline_tune(ctx, C.byref(m), layers, C.byref(batch), *_ws(ws), C.byref(space), C.byref(best),
                                   pts, max_points, C.byref(n), stream_handle(stream)))
    return best, [pts[i] for i in range(min(n.value, max_points))]


# ----------------------------------------------------------------------- schedule model
def spa_sched_binding(k: int, K: int, w: int) -> int:
    return int(lib().spa_sched_binding(k, K, w))


def spa_sched_makespan(n_regions, n_micro, K, w, tau):
    n = n_regions * n_micro * K
    t = (C.c_double * n)(*[float(v) for v in tau])
    st = (C.c_double * n)()
    en = (C.c_double * n)()
    T = C.c_double()
    _check(lib().spa_sched_makespan(n_regions, n_micro, K, w, t, C.byref(T), st, en))
    return T.value, list(st), list(en)


def spa_sched_counts(n_ops, n_stages, n_units, quantum):
    a = C.c_int64()
    b = C.c_int64()
    _check(lib().spa_sched_counts(n_ops, n_stages, n_units, quantum, C.byref(a), C.byref(b)))
    return a.value, b.value


def spa_refine_allocation(n_stages, total, quantum, p_min, p0, objective, pass_limit=0):
    """objective: python callable(tuple) -> float."""
    arr = (C.c_int32 * n_stages)(*p0)

    def _cb(p, n, user):
        return float(objective(tuple(p[i] for i in range(n))))

    cb = OBJECTIVE_FN(_cb)
    best = C.c_double()
    ev = C.c_int32()
    _check(lib().spa_refine_allocation(n_stages, total, quantum, p_min, arr, cb, None, pass_limit, C.byref(best),
                                       C.byref(ev)))
    return tuple(arr), best.value, ev.value
