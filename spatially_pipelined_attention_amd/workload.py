"""Device-resident synthetic workloads: weights, KV caches and the batch.

Builds every input of a decode iteration in HBM from the seeded generator
(synth), plans the packed KV layout (per-sequence capacity rounded up to 32
positions) and writes the cached history through the library's own KV row
I/O, so the device bits equal what the host generator gives the CPU
reference. Input preparation only: no step of the layer runs here.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional

import numpy as np
import torch

from . import binding as B
from . import synth

_DT = {"f32": B.SPA_F32, "bf16": B.SPA_BF16, "e4m3": B.SPA_E4M3}
_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def model_desc(wl: synth.Workload) -> B.spa_model_desc:
    m = B.spa_model_desc(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_experts, wl.n_resident,
                         wl.top_k, wl.inter, wl.window, wl.n_layers, wl.eps, _DT[wl.w_dtype],
                         _DT[wl.expert_dtype], _DT[wl.kv_dtype])
    m.rope_theta = float(wl.rope_theta)
    return m


def set_comm(m: B.spa_model_desc, latency_us: float, gbps: float) -> B.spa_model_desc:
    """Give the model the virtual communication endpoints of one rank (the
    all-reduce after the output projection, MoE dispatch and combine), each
    lasting latency_us + payload bytes / gbps; gbps = 0 removes them. Set it
    before sizing a workspace or creating a pipeline: both copy the model."""
    m.comm_latency_us = float(latency_us)
    m.comm_gbps = float(gbps)
    return m


def parse_comm(spec: str):
    """'LATENCY_US,GBPS' -> (latency_us, gbps); '' or None -> None."""
    if not spec:
        return None
    lat, gbps = (float(v) for v in spec.split(","))
    return lat, gbps


def round_up(v, a):
    return (v + a - 1) // a * a


class DeviceWorkload:
    """All device tensors of one workload and the C descriptors pointing at them."""

    def __init__(self, wl: synth.Workload, resample: Optional[Dict[int, int]] = None, device: str = "cuda",
                 fill_history: bool = True, record_topk: bool = True):
        self.wl = wl
        self.dev = torch.device(device)
        self.m = model_desc(wl)
        self.L = synth.kv_lengths(wl).astype(np.int64)
        self.cap = np.array([round_up(int(l), 32) for l in self.L], np.int64)
        self.off = np.concatenate([[0], np.cumsum(self.cap)[:-1]]).astype(np.int64)
        self.total_cap = int(self.cap.sum())
        self.max_kv_len = int(self.L.max())
        self.kv_len_d = torch.as_tensor(self.L.astype(np.int32), device=self.dev)
        self.kv_off_d = torch.as_tensor(self.off, device=self.dev)
        self.kv_cap_d = torch.as_tensor(self.cap.astype(np.int32), device=self.dev)
        self.resample = dict(resample or {})
        self.x0 = torch.as_tensor(synth.x_rows(wl, list(range(wl.batch)), self.resample), device=self.dev)
        self.x = self.x0.clone()
        self.topk = (torch.zeros((wl.n_layers, wl.batch, wl.top_k), dtype=torch.int32, device=self.dev)
                     if record_topk else None)
        self.layers_t: List[dict] = []
        self.layers_c = (B.spa_layer * wl.n_layers)()
        self._keep = []
        for l in range(wl.n_layers):
            self._build_layer(l, fill_history)
        torch.cuda.synchronize()
        self.batch = B.spa_batch(wl.batch, self.max_kv_len, self.kv_len_d.data_ptr(), self.kv_off_d.data_ptr(),
                                 self.kv_cap_d.data_ptr(), self.x.data_ptr(),
                                 self.topk.data_ptr() if self.topk is not None else None)

    # ------------------------------------------------------------------ build
    def _fill(self, shape, dtype: str, tag: int, layer: int, sub: int, std: float):
        t = torch.empty(shape, dtype=_TORCH[dtype], device=self.dev)
        synth.dev_fill_normal(t, synth.stream_key(self.wl.seed, tag, layer, sub), 0, std)
        return t

    def _pack(self, t: torch.Tensor, dtype: str, n_mats: int, n_rows: int, k: int) -> torch.Tensor:
        """Row-major weight matrices -> the library's panel layout (a byte tensor)."""
        code = _DT[dtype]
        dst = torch.empty(B.spa_packed_bytes(code, n_mats, n_rows, k), dtype=torch.uint8, device=self.dev)
        B.spa_pack_weights(self.ctx_for_io(), code, n_mats, n_rows, k, t, dst, torch.cuda.current_stream())
        return dst

    def _build_layer(self, l: int, fill_history: bool):
        wl = self.wl
        H, I, E, Er = wl.hidden, wl.inter, wl.n_experts, wl.n_resident
        D, Hkv, Hq = wl.head_dim, wl.n_kv_heads, wl.n_q_heads
        t: dict = {}
        t["wqkv"] = self._pack(self._fill((wl.qkv_rows, H), wl.w_dtype, synth.TAG_WQKV, l, 0, wl.w_std),
                               wl.w_dtype, 1, wl.qkv_rows, H)
        t["wo"] = self._pack(self._fill((H, Hq * D), wl.w_dtype, synth.TAG_WO, l, 0, wl.w_std), wl.w_dtype, 1, H, Hq * D)
        t["wr"] = self._pack(self._fill((E, H), "f32", synth.TAG_WR, l, 0, wl.router_sigma), "f32", 1, E, H)
        t["sinks"] = self._fill((Hq,), "f32", synth.TAG_SINK, l, 0, 1.0)
        t["gamma1"] = torch.ones(H, dtype=torch.float32, device=self.dev)
        t["gamma2"] = torch.ones(H, dtype=torch.float32, device=self.dev)
        if wl.expert_dtype == "e4m3":
            gu_c = torch.empty((Er, 2 * I, H), dtype=torch.uint8, device=self.dev)
            d_c = torch.empty((Er, H, I), dtype=torch.uint8, device=self.dev)
            gu_s = torch.empty((Er, 2 * I), dtype=torch.float32, device=self.dev)
            d_s = torch.empty((Er, H), dtype=torch.float32, device=self.dev)
            for e in range(Er):
                ew = synth.expert_weights(wl, l, e)
                gu_c[e].copy_(torch.from_numpy(ew["wgu_codes"]))
                d_c[e].copy_(torch.from_numpy(ew["wd_codes"]))
                gu_s[e].copy_(torch.from_numpy(ew["wgu_scale"]))
                d_s[e].copy_(torch.from_numpy(ew["wd_scale"]))
            t.update(wgu=self._pack(gu_c, "e4m3", Er, 2 * I, H), wd=self._pack(d_c, "e4m3", Er, H, I),
                     wgu_scale=gu_s, wd_scale=d_s)
        else:
            wgu = torch.empty((Er, 2 * I, H), dtype=_TORCH[wl.expert_dtype], device=self.dev)
            wd = torch.empty((Er, H, I), dtype=_TORCH[wl.expert_dtype], device=self.dev)
            for e in range(Er):
                synth.dev_fill_normal(wgu[e], synth.stream_key(wl.seed, synth.TAG_WGU, l, e), 0, wl.w_std)
                synth.dev_fill_normal(wd[e], synth.stream_key(wl.seed, synth.TAG_WD, l, e), 0, wl.w_std)
            t.update(wgu=self._pack(wgu, wl.expert_dtype, Er, 2 * I, H), wd=self._pack(wd, wl.expert_dtype, Er, H, I),
                     wgu_scale=None, wd_scale=None)
        kind = wl.layer_kinds[l]
        kvt = _TORCH[wl.kv_dtype]
        if kind == "full":
            n_el = self.total_cap * Hkv * D
        else:
            n_el = wl.batch * Hkv * wl.window * D
        t["k_cache"] = torch.zeros(n_el, dtype=kvt, device=self.dev)
        t["v_cache"] = torch.zeros(n_el, dtype=kvt, device=self.dev)
        t["kind"] = B.SPA_FULL if kind == "full" else B.SPA_SLIDING
        self.layers_t.append(t)
        c = self.layers_c[l]
        c.kind = t["kind"]
        for name in ("wqkv", "wo", "wr", "wgu", "wd", "wgu_scale", "wd_scale", "gamma1", "gamma2", "sinks",
                     "k_cache", "v_cache"):
            setattr(c, name, B.ptr(t[name]))
        if fill_history:
            self._fill_history(l)

    def history_rows(self, l: int, seqs=None):
        """(seq, pos) of every cached history position of layer l (positions before L-1 in the window)."""
        seqs = range(self.wl.batch) if seqs is None else seqs
        ss, pp = [], []
        for b in seqs:
            lo, hi = synth.history_range(self.wl, l, int(self.L[b]))
            if hi > lo:
                ss.append(np.full(hi - lo, b, np.int32))
                pp.append(np.arange(lo, hi, dtype=np.int32))
        if not ss:
            return np.zeros(0, np.int32), np.zeros(0, np.int32)
        return np.concatenate(ss), np.concatenate(pp)

    def _fill_history(self, l: int, chunk_rows: int = 1 << 18):
        wl = self.wl
        seq, pos = self.history_rows(l)
        Hkv, D = wl.n_kv_heads, wl.head_dim
        kvt = _TORCH[wl.kv_dtype]
        kkey = synth.stream_key(wl.seed, synth.TAG_KHIST, l)
        vkey = synth.stream_key(wl.seed, synth.TAG_VHIST, l)
        t = self.layers_t[l]
        for r0 in range(0, len(seq), chunk_rows):
            s = seq[r0:r0 + chunk_rows]
            p = pos[r0:r0 + chunk_rows]
            n = len(s)
            g = np.arange(Hkv, dtype=np.int64)
            bases = ((((s.astype(np.int64)[:, None] * Hkv + g[None, :]) << synth.KV_POS_BITS)
                      + p.astype(np.int64)[:, None]) * D).reshape(-1)
            kr = torch.empty((n * Hkv, D), dtype=kvt, device=self.dev)
            vr = torch.empty((n * Hkv, D), dtype=kvt, device=self.dev)
            kb = synth.dev_fill_rows(kr, bases, kkey, 1.0)
            vb = synth.dev_fill_rows(vr, bases, vkey, 1.0)
            sd = torch.as_tensor(s, device=self.dev)
            pd = torch.as_tensor(p, device=self.dev)
            B.spa_kv_io(self.ctx_for_io(), self.m, t["kind"], t["k_cache"], t["v_cache"], self._io_batch(), sd, pd, n,
                        kr, vr, 1)
            torch.cuda.synchronize()
            del kb, vb

    _io_ctx = None

    @classmethod
    def ctx_for_io(cls):
        if cls._io_ctx is None:
            cls._io_ctx = B.spa_init(0)
        return cls._io_ctx

    def _io_batch(self):
        return B.spa_batch(self.wl.batch, self.max_kv_len, self.kv_len_d.data_ptr(), self.kv_off_d.data_ptr(),
                           self.kv_cap_d.data_ptr(), self.x.data_ptr(), None)

    # ------------------------------------------------------------------ helpers
    def reset_x(self):
        self.x.copy_(self.x0)

    def read_kv(self, l: int, seqs, positions):
        """Cached K, V at (seq, pos) pairs -> float32 numpy [n][Hkv][D]."""
        wl = self.wl
        n = len(seqs)
        kvt = _TORCH[wl.kv_dtype]
        kr = torch.empty((n, wl.n_kv_heads, wl.head_dim), dtype=kvt, device=self.dev)
        vr = torch.empty_like(kr)
        t = self.layers_t[l]
        B.spa_kv_io(self.ctx_for_io(), self.m, t["kind"], t["k_cache"], t["v_cache"], self._io_batch(),
                    torch.as_tensor(np.asarray(seqs, np.int32), device=self.dev),
                    torch.as_tensor(np.asarray(positions, np.int32), device=self.dev), n, kr, vr, 0)
        torch.cuda.synchronize()
        return kr.float().cpu().numpy(), vr.float().cpu().numpy()

    def workspace(self, n_micro: int = 1, n_tok: Optional[int] = None) -> torch.Tensor:
        if n_tok is None:
            nb = B.spa_workspace_query(self.m, self.wl.batch, self.max_kv_len, n_micro)
        else:
            nb = B.spa_workspace_query(self.m, n_tok, self.max_kv_len, 1)
        return torch.empty(nb + 256, dtype=torch.uint8, device=self.dev)

    def algorithmic_kv_bytes(self, l: int) -> int:
        """Bytes of K and V one decode step of layer l must read (attended window)."""
        wl = self.wl
        esz = 2 if wl.kv_dtype == "bf16" else 4
        tot = 0
        for b in range(wl.batch):
            n = min(int(self.L[b]), wl.window) if wl.layer_kinds[l] == "sliding" else int(self.L[b])
            tot += n * wl.n_kv_heads * wl.head_dim * esz * 2
        return tot


class Pipeline:
    """A pipeline (and the CU pools it owns) from a configuration dict:
    {"cut", "n_micro", "cu_a"[, "cu_a_sliding", "handoff", "graph", "head"]}; cu_a = None or 0 gives the
    temporal schedule with the same microbatches. Stage A takes the first
    cu_a CUs of every XCD's share, stage B the rest."""

    def __init__(self, ctx, m: B.spa_model_desc, cfg: dict, verify: bool = True):
        self.pools = []
        n_cus = B.spa_device_cus(ctx)
        c = B.spa_pipeline_cfg(int(cfg["cut"]), int(cfg["n_micro"]), int(cfg.get("handoff", 0)), 0,
                               int(cfg.get("head", 0)))
        cu_a = cfg.get("cu_a") or 0
        if cu_a <= 0:
            c.graph = int(cfg.get("graph", 0))   # graph replay: temporal schedules only
            self.h = B.spa_pipeline_create(ctx, m, c, None, None)
            return

        def split(cu):
            pa = B.spa_pool_create_split(ctx, 0, cu)
            self.pools.append(pa)
            pb = B.spa_pool_create_split(ctx, cu // 8, n_cus - cu)
            self.pools.append(pb)
            if verify:   # the kernels must land on the masked CUs, not silently on the whole GPU
                B.spa_pool_verify(pa)
                B.spa_pool_verify(pb)
            return pa, pb
        cu_s = cfg.get("cu_a_sliding") or cu_a
        af, bf = split(cu_a)
        if cu_s == cu_a:
            self.h = B.spa_pipeline_create(ctx, m, c, af, bf)
        else:
            asl, bsl = split(cu_s)
            self.h = B.spa_pipeline_create_kinds(ctx, m, c, af, bf, asl, bsl)

    def run(self, layers, batch, ws, stream=None):
        B.spa_pipeline_run(self.h, layers, batch, ws, stream if stream is not None else torch.cuda.current_stream())

    def close(self):
        B.spa_pipeline_destroy(self.h)
        for p in self.pools:
            B.spa_pool_destroy(p)
        self.pools = []
