"""Host orchestration of the compile and link steps on the HIP path.

This module only plans memory (page allocation through the library's C++
allocator, index arrays) and issues the C-ABI calls in order on one HIP
stream; every step of the method runs in the library's kernels.  Selection
sizes produced on the device (|S_k| after the top-k and after each refresh)
reach the later kernels as device-side row counts; with exact_rows (the
default) the step also reads each new count back (4 bytes) so that later
launches are sized to it.

Token spaces.  Compile: the unique chunk instances concatenated, each its own
segment (positions from 0, keys visible from the chunk start).  Link: the
requests concatenated (token g of request b at position g - cu_tok[b], keys
visible from cu_tok[b]).

Page plan (CacheSlide page, SLIDE implementation paragraph; 16-token pages):
compile pages per chunk instance and layer, then per request and layer the
link's new pages, N_r tokens' worth at layer 1 and floor(ratio * N_r) at later
layers (CacheSlide; cb_ratio for the CacheBlend-style selection), or |S_r| at
every layer (LegoLink).  An uncached query chunk has no compile pages.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Callable, List, Optional

import numpy as np
import torch

from . import _lib as K

PAGE = 16


def _i32(x, device) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=device)


def _cached(chunk) -> bool:
    """A chunk has compile-step KV unless it is the request's uncached query."""
    return getattr(chunk, "kind", "fixed") != "query"


def _npages(n: int) -> int:
    return (int(n) + PAGE - 1) // PAGE


def spill_order(counts, pages) -> List[int]:
    """SLIDE's eviction order of `pages` (CacheSlide page, SLIDE paragraphs:
    clean pages go first, then dirty pages in descending order of their
    selected-token counter); equal counters by lower page id."""
    pages = sorted(int(p) for p in pages)
    clean = [p for p in pages if counts[p] == 0]
    dirty = sorted((p for p in pages if counts[p] != 0), key=lambda p: (-int(counts[p]), p))
    return clean + dirty


class Model:
    """Weights of a decoder stack resident on the device (caller-provided tensors)."""

    def __init__(self, shape, embedding: torch.Tensor, layers: List[dict]):
        self.shape = shape
        self.embedding = embedding
        self.layers = layers


@dataclass
class LinkConfig:
    mode: str = "cacheslide"          # "cacheslide", "legolink" or "cacheblend"
    ratio: float = 0.26               # CacheSlide top-k ratio
    cb_ratio: float = 0.15            # CacheBlend-style top-k ratio
    tau: float = 0.12
    period: int = 4
    lego_k: int = 32
    alpha_mode: int = K.KVB_ALPHA_LAG
    refresh_rule: int = K.KVB_REFRESH_LITERAL
    # After each refresh, read the surviving row count back to the host (a
    # 4-byte copy and one wait) so later layers launch at their true size and
    # layers left with no rows are skipped; False keeps every launch sized for
    # the layer-1 selection.  The device-side count bounds the rows either way.
    exact_rows: bool = True
    # Where the compile step's KV (the reused cache) lives during the link
    # step.  "hbm": resident in the device pool.  "host": in pinned host memory
    # (SLIDE's lower tier); each layer's reused pages are copied into the pool
    # during the step, on a copy stream that runs `tier_lookahead` layers ahead
    # of the recompute (tier_overlap=True) or on the compute stream right before
    # the layer (False: the serial baseline).
    reuse_tier: str = "hbm"
    tier_overlap: bool = True
    tier_lookahead: int = 2


class LinkEngine:
    """Plans and runs the compile and link steps of a batch of requests.

    requests: objects with `.chunks`, each chunk with `.uid` and `.tokens`
    (int array); chunks sharing a uid are compiled once and their pages are
    shared read-only by every request that splices them.
    """

    def __init__(self, model: Model, requests, cfg: LinkConfig, device="cuda:0", stream=None, max_decode: int = 0):
        if cfg.mode != "legolink" and any(not _cached(c) for r in requests for c in r.chunks):
            raise ValueError("uncached query chunks must be recomputed in every layer: use mode='legolink'")
        self.model, self.cfg, self.device = model, cfg, torch.device(device)
        self.requests = list(requests)
        s = model.shape
        self.shape = s
        self.L = s.n_layers
        self.desc = K.model_desc(s)
        self.ctx = K.kvb_create(self.device.index or 0)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.sh = K.stream_handle(self.stream)
        self.tdtype = torch.bfloat16 if s.dtype == "bf16" else torch.float32
        self.scale = 1.0 / math.sqrt(s.head_dim)
        dev = self.device

        # ---------------- token spaces
        chunks, seen = [], set()
        for r in requests:
            for c in r.chunks:
                if _cached(c) and c.uid not in seen:
                    seen.add(c.uid)
                    chunks.append(c)
        self.chunks = chunks
        self.B = len(requests)
        lens_c = [len(c.tokens) for c in chunks]
        self.Nc = int(sum(lens_c))
        cu_c = np.concatenate([[0], np.cumsum(lens_c)]).astype(np.int64)
        self.req_lens = [int(sum(len(c.tokens) for c in r.chunks)) for r in requests]
        self.N = int(sum(self.req_lens))
        cu_t = np.concatenate([[0], np.cumsum(self.req_lens)]).astype(np.int64)
        self.cu_tok_h = cu_t
        tok_c = np.concatenate([np.asarray(c.tokens, dtype=np.int32) for c in chunks])
        tok_l = np.concatenate([np.asarray(c.tokens, dtype=np.int32) for r in requests for c in r.chunks])
        pos_c = np.concatenate([np.arange(n) for n in lens_c])
        lo_c = np.concatenate([np.full(n, cu_c[i]) for i, n in enumerate(lens_c)])
        pos_l = np.concatenate([np.arange(n) for n in self.req_lens])
        lo_l = np.concatenate([np.full(n, cu_t[b]) for b, n in enumerate(self.req_lens)])

        # ---------------- page plan (host allocator in the library)
        if cfg.mode in ("cacheslide", "cacheblend"):
            ratio = cfg.ratio if cfg.mode == "cacheslide" else cfg.cb_ratio
            self.k_cap = [int(math.floor(ratio * n)) for n in self.req_lens]
            per_layer = lambda l, b: self.req_lens[b] if l == 1 else self.k_cap[b]
        elif cfg.mode == "legolink":
            rows = []
            for r, start in zip(requests, cu_t[:-1]):
                s0 = 0
                rr = []
                for ci, c in enumerate(r.chunks):
                    if not _cached(c):       # the query: all of it, in every layer
                        rr.extend(range(s0, s0 + len(c.tokens)))
                    elif ci > 0:
                        rr.extend(range(s0, s0 + min(cfg.lego_k, len(c.tokens))))
                    s0 += len(c.tokens)
                rows.append(np.asarray(rr, dtype=np.int64) + start)
            self.lego_rows = rows
            self.k_cap = [len(x) for x in rows]
            per_layer = lambda l, b: self.k_cap[b]
        else:
            raise ValueError(cfg.mode)
        n_compile_pages = sum(_npages(n) for n in lens_c) * self.L
        n_link_pages = sum(_npages(per_layer(l, b)) for l in range(1, self.L + 1) for b in range(self.B))
        # decode continuation: room for max_decode tokens per request and layer
        # when no overwritable slot is left (allocated after every other page)
        self.max_decode = int(max_decode)
        n_decode_pages = _npages(self.max_decode) * self.L * self.B if self.max_decode > 0 else 0
        self.n_pages = n_compile_pages + n_link_pages + n_decode_pages
        self.pool = K.kvb_pool_create(self.n_pages)
        comp_pages = {}
        for c in chunks:
            comp_pages[c.uid] = [K.kvb_pool_alloc(self.pool, _npages(len(c.tokens))) for _ in range(self.L)]
        link_pages = [[None] * (self.L + 1) for _ in range(self.B)]
        for b in range(self.B):
            for l in range(1, self.L + 1):
                link_pages[b][l] = K.kvb_pool_alloc(self.pool, _npages(per_layer(l, b)))
        self.comp_pages, self.link_pages = comp_pages, link_pages
        # compile pages are the first n_compile_pages ids; per layer, those every
        # request may read (reused K/V of that layer)
        self.n_compile_pages = n_compile_pages
        self.layer_reuse_pages = [None] + [
            sorted(p for c in chunks for p in comp_pages[c.uid][l - 1]) for l in range(1, self.L + 1)]

        def slots(pages, n):
            j = np.arange(n)
            return np.asarray(pages, dtype=np.int64)[j // PAGE] * PAGE + j % PAGE

        comp_slot = np.zeros((self.L, self.Nc), dtype=np.int32)
        for i, c in enumerate(chunks):
            for l in range(self.L):
                comp_slot[l, cu_c[i]:cu_c[i + 1]] = slots(comp_pages[c.uid][l], len(c.tokens))
        reuse_slot = np.zeros((self.L, self.N), dtype=np.int32)
        for b, r in enumerate(requests):
            g = cu_t[b]
            for c in r.chunks:
                n = len(c.tokens)
                for l in range(self.L):
                    reuse_slot[l, g:g + n] = slots(comp_pages[c.uid][l], n) if _cached(c) else -1
                g += n
        self.comp_slot_h, self.reuse_slot_h = comp_slot, reuse_slot
        new_pages, cu_pages = [None], [None]
        for l in range(1, self.L + 1):
            pl = [link_pages[b][l] for b in range(self.B)]
            new_pages.append(_i32(np.concatenate([np.asarray(p, dtype=np.int64) for p in pl]) if sum(map(len, pl))
                                  else np.zeros(1), dev))
            cu_pages.append(_i32(np.concatenate([[0], np.cumsum([len(p) for p in pl])]), dev))
        self.new_pages, self.cu_pages = new_pages, cu_pages

        # ---------------- device arrays
        self.tok_c = _i32(tok_c, dev)
        self.tok_l = _i32(tok_l, dev)
        self.pos_c, self.lo_c = _i32(pos_c, dev), _i32(lo_c, dev)
        self.pos_l, self.lo_l = _i32(pos_l, dev), _i32(lo_l, dev)
        self.cu_tok = _i32(cu_t, dev)
        self.comp_slot = _i32(comp_slot, dev)
        self.reuse_slot = _i32(reuse_slot, dev)
        self.k_cap_d = _i32(self.k_cap, dev)
        self.T_sel = int(sum(self.k_cap))
        if cfg.mode == "legolink":
            sel = np.concatenate(self.lego_rows) if self.T_sel else np.zeros(1)
            self.lego_sel = _i32(sel, dev)
            self.lego_cu = _i32(np.concatenate([[0], np.cumsum(self.k_cap)]), dev)

        # ---------------- buffers
        d, Hq, Hkv, hd = s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim
        rows_max = max(self.Nc, self.N, 1)
        td = self.tdtype
        self.k_pool = torch.zeros((self.n_pages, Hkv, PAGE, hd), dtype=td, device=dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.hidden_c = torch.zeros((max(self.Nc, 1), d), dtype=td, device=dev)
        self.hidden = torch.zeros((max(self.N, 1), d), dtype=td, device=dev)
        self.q = torch.empty((rows_max, Hq, hd), dtype=td, device=dev)
        self.k = torch.empty((rows_max, Hkv, hd), dtype=td, device=dev)
        self.v = torch.empty((rows_max, Hkv, hd), dtype=td, device=dev)
        self.o = torch.empty((rows_max, Hq * hd), dtype=td, device=dev)
        nt = max(self.N, 1)
        self.alpha = torch.zeros(nt, dtype=torch.float32, device=dev)
        self.d = torch.zeros(nt, dtype=torch.float32, device=dev)
        self.ranking = torch.zeros(nt, dtype=torch.int32, device=dev)
        self.s_count = torch.zeros(self.B, dtype=torch.int32, device=dev)
        self.cursor = torch.zeros(self.B, dtype=torch.int32, device=dev)
        self.sel = [torch.zeros(nt, dtype=torch.int32, device=dev) for _ in range(2)]
        self.cu_rows = [torch.zeros(self.B + 1, dtype=torch.int32, device=dev) for _ in range(2)]
        self.dev_l = torch.zeros(max(self.T_sel, 1), dtype=torch.float32, device=dev)
        self.cksim = torch.zeros(max(self.T_sel, 1), dtype=torch.float32, device=dev)
        # per-layer page table of the link step: the slot of every token's K/V in
        # that layer (reused slot, or the new slot of a recomputed row)
        self.page_table = torch.zeros((self.L, nt), dtype=torch.int32, device=dev)
        self.slot_map = self.page_table[0]  # the layer being run
        self._pt_reuse_rows = set()         # layers skipped by the last step: their rows still to fill
        self.dst_slot = torch.zeros(rows_max, dtype=torch.int32, device=dev)
        # SLIDE's dirty-page counters: selected tokens routed into each page from
        # layer 2 on, then the decode tokens written into it (cleared per link step)
        self.page_dirty = torch.zeros(self.n_pages, dtype=torch.int32, device=dev)
        self.ws_bytes = K.kvb_workspace_size(self.ctx, self.desc, rows_max, max(self.N, self.Nc), self.B)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.cur = 0
        self._count_h = torch.zeros(1, dtype=torch.int32, pin_memory=True)
        self._count_ev = torch.cuda.Event()

    # ------------------------------------------------------------------ helpers
    def close(self):
        if getattr(self, "pool", None) is not None:
            K.kvb_pool_destroy(self.pool)
            self.pool = None
        if getattr(self, "ctx", None) is not None:
            K.kvb_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _n_rows_ptr(self, which: int) -> int:
        return self.cu_rows[which].data_ptr() + 4 * self.B

    def _start_read_rows(self, which: int):
        """Queue the copy of selection buffer `which`'s total row count to the host
        at this point of the engine stream."""
        with torch.cuda.stream(self.stream):
            self._count_h.copy_(self.cu_rows[which][self.B:self.B + 1], non_blocking=True)
            self._count_ev.record(self.stream)

    def _finish_read_rows(self) -> int:
        self._count_ev.synchronize()
        return int(self._count_h[0])

    def _read_rows(self, which: int) -> int:
        """Total rows of selection buffer `which`, copied to the host once the
        engine stream reaches this point."""
        self._start_read_rows(which)
        return self._finish_read_rows()

    # ------------------------------------------------------------------ compile step
    def run_compile(self):
        """Prefill every chunk instance alone from position 0 into its compile pages."""
        c, sh, ds, Nc = self.ctx, self.sh, self.desc, self.Nc
        if Nc == 0:
            return
        m = self.model
        K.kvb_embed(c, sh, ds, Nc, None, None, self.tok_c, self.shape.vocab, m.embedding, self.hidden_c)
        for l in range(1, self.L + 1):
            W = m.layers[l - 1]
            K.kvb_qkv_fused(c, sh, ds, Nc, None, None, self.hidden_c, W["norm1"], W["w_qkv"], self.pos_c,
                            self.q, self.k, self.v, self.k_pool, self.v_pool, self.n_pages, None,
                            self.comp_slot[l - 1], K.KVB_ALPHA_ONE, None, None, None, self.ws, self.ws_bytes)
            if l < self.L:
                K.kvb_sparse_query_attn(c, sh, ds, Nc, None, None, self.lo_c, self.q, self.k_pool, self.v_pool,
                                        self.n_pages, self.comp_slot[l - 1], self.scale, self.o, self.ws,
                                        self.ws_bytes)
                K.kvb_mlp(c, sh, ds, Nc, None, None, self.o, W["w_o"], self.hidden_c, W["norm2"], W["w_gate_up"],
                          W["w_down"], self.ws, self.ws_bytes)

    def stage_reuse_to_host(self, evict: bool = False):
        """Copy the compile pages to pinned host memory (the lower tier the link
        step then loads from).  evict=True also zeroes their device copies, so a
        link step can only see what it loads."""
        if self.cfg.reuse_tier != "host":
            raise ValueError("stage_reuse_to_host needs reuse_tier='host'")
        n = self.n_compile_pages
        if getattr(self, "host_k", None) is None:
            shp = (max(n, 1),) + tuple(self.k_pool.shape[1:])
            self.host_k = torch.empty(shp, dtype=self.k_pool.dtype, pin_memory=True)
            self.host_v = torch.empty(shp, dtype=self.v_pool.dtype, pin_memory=True)
        K.kvb_pages_copy(self.ctx, self.sh, self.desc, K.KVB_COPY_D2H, self.k_pool, self.v_pool, self.host_k,
                         self.host_v, range(n))
        self.stream.synchronize()
        if evict and n:
            with torch.cuda.stream(self.stream):
                self.k_pool[:n].zero_()
                self.v_pool[:n].zero_()
            self.stream.synchronize()

    # ------------------------------------------------------------------ tiers
    def _tier_begin(self):
        """Start of a link step that loads its reused pages from the host tier."""
        self._tier = self.cfg.reuse_tier == "host"
        if not self._tier:
            return
        if getattr(self, "host_k", None) is None:
            raise RuntimeError("reuse_tier='host': call stage_reuse_to_host() after run_compile()")
        self._tier_enq = 0
        self._tier_ev = [None] * (self.L + 1)
        self._tier_loaded = {}   # layer -> "k" or "kv": what this step copied in
        if self.cfg.tier_overlap:
            if getattr(self, "copy_stream", None) is None:
                self.copy_stream = torch.cuda.Stream(self.device)  # default priority
            start = torch.cuda.Event()
            start.record(self.stream)
            self.copy_stream.wait_event(start)  # the previous step is done with the pool

    def _tier_copy(self, l: int, stream_handle: int, keys_only: Optional[bool] = None):
        # layer 1 of CacheSlide and of the CacheBlend-style link reads reused keys
        # only (the deviation compares keys)
        if keys_only is None:
            keys_only = l == 1 and self.cfg.mode != "legolink"
        K.kvb_pages_copy(self.ctx, stream_handle, self.desc, K.KVB_COPY_H2D, self.host_k,
                         None if keys_only else self.host_v, self.k_pool, None if keys_only else self.v_pool,
                         self.layer_reuse_pages[l])
        self._tier_loaded[l] = "k" if keys_only else "kv"

    def _tier_fill_for_decode(self, pt: np.ndarray):
        """Before decode: copy in the reused K/V of every layer whose page table
        still points at reused slots but whose pages the last link step did not
        load (layers it skipped, or loaded keys only), so decode never attends
        over an evicted page."""
        if self.cfg.reuse_tier != "host" or getattr(self, "host_k", None) is None:
            return
        loaded = getattr(self, "_tier_loaded", {})
        for l in range(1, self.L + 1):
            if loaded.get(l) == "kv":
                continue
            rs = self.reuse_slot_h[l - 1]
            if np.any((pt[l - 1] == rs) & (rs >= 0)):
                self._tier_copy(l, self.sh, keys_only=False)

    def _tier_need(self, l: int, runs_until: int):
        """Before layer l: its reused pages are in the pool.  Layers up to
        runs_until are known to run, so copies for them may be queued ahead."""
        if not self._tier:
            return
        if not self.cfg.tier_overlap:
            self._tier_copy(l, self.sh)
            return
        last = min(self.L, runs_until, l + self.cfg.tier_lookahead)
        ch = K.stream_handle(self.copy_stream)
        while self._tier_enq < max(last, l):
            j = self._tier_enq + 1
            self._tier_copy(j, ch)
            ev = torch.cuda.Event()
            ev.record(self.copy_stream)
            self._tier_ev[j] = ev
            self._tier_enq = j
        self.stream.wait_event(self._tier_ev[l])

    def _tier_end(self):
        # copies queued ahead for layers that were then skipped belong to this step
        if self._tier and self.cfg.tier_overlap and self._tier_enq:
            self.stream.wait_event(self._tier_ev[self._tier_enq])

    # ------------------------------------------------------------------ link step
    def run_link(self, hook: Optional[Callable] = None):
        self._pt_reuse_rows = set()
        with torch.cuda.stream(self.stream):
            self.page_dirty.zero_()
        self._tier_begin()
        if self.cfg.mode == "cacheslide":
            self._link_cacheslide(hook)
        elif self.cfg.mode == "cacheblend":
            self._link_cacheblend(hook)
        else:
            self._link_static(hook)
        self._tier_end()

    def link_desc(self) -> "K.kvb_link_desc":
        """The kvb_link_desc of this engine's link step (the reused cache
        resident in the pool).  The host arrays it points to are kept on the
        engine."""
        if self.cfg.reuse_tier != "hbm":
            raise ValueError("kvb_link_run reads the reused cache from the device pool")
        L, mode = self.L, self.cfg.mode
        cs = mode == "cacheslide"
        lw = (K.kvb_layer_weights * L)()
        for i, W in enumerate(self.model.layers):
            lw[i] = K.kvb_layer_weights(W["norm1"].data_ptr(), W["w_qkv"].data_ptr(), W["w_o"].data_ptr(),
                                        W["norm2"].data_ptr(), W["w_gate_up"].data_ptr(), W["w_down"].data_ptr())
        npg = (ctypes.c_void_p * L)(*[self.new_pages[l].data_ptr() for l in range(1, L + 1)])
        cpg = (ctypes.c_void_p * L)(*[self.cu_pages[l].data_ptr() for l in range(1, L + 1)])
        self._link_host = (lw, npg, cpg)
        t = lambda x: x.data_ptr() if x is not None else None
        k = K.kvb_link_desc()
        k.mode = {"cacheslide": K.KVB_LINK_CACHESLIDE, "legolink": K.KVB_LINK_STATIC,
                  "cacheblend": K.KVB_LINK_CACHEBLEND}[mode]
        k.B, k.n_tok, k.n_layers, k.n_pages, k.vocab = self.B, self.N, L, self.n_pages, self.shape.vocab
        k.rows, k.period, k.refresh_rule, k.alpha_mode = self.T_sel, self.cfg.period, self.cfg.refresh_rule, \
            self.cfg.alpha_mode
        k.tau, k.scale = float(self.cfg.tau), float(self.scale)
        k.layers = ctypes.addressof(lw)
        k.embedding, k.tokens, k.pos, k.lo = t(self.model.embedding), t(self.tok_l), t(self.pos_l), t(self.lo_l)
        k.cu_tok, k.reuse_slot = t(self.cu_tok), t(self.reuse_slot)
        k.k_cap = t(self.k_cap_d) if mode != "legolink" else None
        k.new_pages, k.cu_pages = ctypes.addressof(npg), ctypes.addressof(cpg)
        if mode == "legolink":
            k.static_rows, k.static_cu = t(self.lego_sel), t(self.lego_cu)
        k.page_table, k.k_pool, k.v_pool, k.hidden = t(self.page_table), t(self.k_pool), t(self.v_pool), t(self.hidden)
        k.q, k.k, k.v, k.o = t(self.q), t(self.k), t(self.v), t(self.o)
        k.d, k.alpha, k.dev, k.cksim = t(self.d), t(self.alpha), t(self.dev_l), t(self.cksim)
        k.ranking, k.s_count, k.cursor = t(self.ranking), t(self.s_count), t(self.cursor)
        k.sel[0], k.sel[1] = t(self.sel[0]), t(self.sel[1])
        k.cu_rows[0], k.cu_rows[1] = t(self.cu_rows[0]), t(self.cu_rows[1])
        k.dst_slot, k.page_dirty, k.ws, k.ws_bytes = t(self.dst_slot), t(self.page_dirty), t(self.ws), self.ws_bytes
        return k

    def run_link_native(self, link_desc=None):
        """The link step as one library call (kvb_link_run): the same steps as
        run_link with exact_rows=False, queued by the library's C++ layer loop
        with no host synchronisation (so it can be recorded in a HIP graph)."""
        k = link_desc if link_desc is not None else self.link_desc()
        self._pt_reuse_rows = set()
        self.cur = K.kvb_link_run(self.ctx, self.sh, self.desc, k)

    def _layer_rows(self, l, T, n_rows, rows, cu_rows, src_slot, alpha_mode, alpha, d_out, cksim_out,
                    after_blend=None):
        """One recompute layer for the given rows: slot map, Q/K/V + RoPE, fusion and
        scatter into new pages, attention over the spliced KV, O-proj + MLP.
        `after_blend` (optional) queues more work right after the fusion."""
        c, sh, ds, W = self.ctx, self.sh, self.desc, self.model.layers[l - 1]
        self.slot_map = self.page_table[l - 1]
        K.kvb_slot_map(c, sh, ds, self.B, self.N, T, cu_rows, rows, self.reuse_slot[l - 1], self.new_pages[l],
                       self.cu_pages[l], self.slot_map, self.dst_slot, self.n_pages,
                       self.page_dirty if l >= 2 else None)
        # layer 1's keys must be bitwise those of the compile step (chunk 0 deviates by
        # exactly 0): batch-invariant there; the selective layers may split K
        flags = K.KVB_QKV_BATCH_INVARIANT if l == 1 else K.KVB_QKV_SPLIT_K
        # projection, RoPE, fusion with the cached rows and scatter to the new slots
        K.kvb_qkv_fused(c, sh, ds, T, n_rows, rows, self.hidden, W["norm1"], W["w_qkv"], self.pos_l, self.q,
                        self.k, self.v, self.k_pool, self.v_pool, self.n_pages, src_slot, self.dst_slot, alpha_mode,
                        alpha, d_out, cksim_out, self.ws, self.ws_bytes, flags)
        if after_blend:
            after_blend()
        K.kvb_sparse_query_attn(c, sh, ds, T, n_rows, rows, self.lo_l, self.q, self.k_pool, self.v_pool,
                                self.n_pages, self.slot_map, self.scale, self.o, self.ws, self.ws_bytes)
        K.kvb_mlp(c, sh, ds, T, n_rows, rows, self.o, W["w_o"], self.hidden, W["norm2"], W["w_gate_up"],
                  W["w_down"], self.ws, self.ws_bytes)

    def _link_cacheslide(self, hook):
        c, sh, ds, N, B = self.ctx, self.sh, self.desc, self.N, self.B
        cfg = self.cfg
        K.kvb_embed(c, sh, ds, N, None, None, self.tok_l, self.shape.vocab, self.model.embedding, self.hidden)
        # layer 1: every token recomputed at its spliced position, written to layer-1 new pages
        self._layer_rows(1, N, None, None, self.cu_tok, None, K.KVB_ALPHA_ONE, None, None, None)
        self._tier_need(1, min(self.L, cfg.period + 1))
        K.kvb_deviation_topk(c, sh, ds, B, N, self.cu_tok, self.k, self.k_pool, self.n_pages, self.reuse_slot[0],
                             self.k_cap_d, self.d, self.alpha, self.ranking, self.s_count, self.sel[0],
                             self.cu_rows[0], self.cursor, self.ws, self.ws_bytes)
        self.cur = 0
        if hook:
            hook(1, self)
        T = self.T_sel
        exact = cfg.exact_rows
        for l in range(2, self.L + 1):
            cur = self.cur
            if T == 0:
                # no row left to recompute: this layer's new pages stay unused and
                # its page table is the reused slots (filled on demand)
                self._pt_reuse_rows.add(l)
                if hook:
                    hook(l, self)
                continue
            refresh = (l % cfg.period == 0) and l < self.L
            # every layer up to the next refresh runs with the current set; the
            # layer after it is loaded speculatively (it runs unless the refresh
            # empties the set, and then its load is only wasted transfer)
            self._tier_need(l, -(-l // cfg.period) * cfg.period + 1 if exact else self.L)
            # the device count always bounds the rows: until the first refresh T is
            # the capacity, which the top-k does not fill when few tokens deviate
            # The refresh needs only this layer's cosine similarities, which the
            # fusion writes, and it fills the other selection buffer, so it can run
            # right after the fusion: the row count then reaches the host while the
            # layer's attention and MLP still run.  With a hook (which inspects the
            # state layer by layer) it runs after the layer; the results are the same.
            def refresh_now(cur=cur, T=T):
                K.kvb_cosine_refresh(c, sh, ds, B, N, self.cu_tok, T, self.cu_rows[cur], self.sel[cur], self.cksim,
                                     cfg.tau, cfg.refresh_rule, self.ranking, self.s_count, self.cursor,
                                     self.sel[1 - cur], self.cu_rows[1 - cur], self.ws, self.ws_bytes)
                if exact:
                    self._start_read_rows(1 - cur)

            early = refresh and hook is None
            self._layer_rows(l, T, self._n_rows_ptr(cur), self.sel[cur], self.cu_rows[cur], self.reuse_slot[l - 1],
                             cfg.alpha_mode, self.alpha, self.dev_l, self.cksim if refresh else None,
                             after_blend=refresh_now if early else None)
            if hook:
                hook(l, self)
            if refresh:
                if not early:
                    refresh_now()
                self.cur = 1 - cur
                if exact:
                    T = self._finish_read_rows()
                if hook:
                    hook(("refresh", l), self)

    def _link_cacheblend(self, hook):
        """CacheBlend-style link (EPIC page, section 3.2): layer 1 recomputes every
        token; each token's attention row under the cached layer-1 keys is
        compared with its row under the recomputed ones, and the cb_ratio share
        that deviates most is recomputed in layers 2..L, its K/V replacing the
        cached ones (no fusion, no refresh)."""
        c, sh, ds, N, B = self.ctx, self.sh, self.desc, self.N, self.B
        K.kvb_embed(c, sh, ds, N, None, None, self.tok_l, self.shape.vocab, self.model.embedding, self.hidden)
        self._layer_rows(1, N, None, None, self.cu_tok, None, K.KVB_ALPHA_ONE, None, None, None)
        self._tier_need(1, self.L)
        # self.q / self.k still hold layer 1's queries and recomputed keys of every token
        K.kvb_attnmap_deviation(c, sh, ds, N, self.lo_l, self.q, self.k, self.k_pool, self.n_pages,
                                self.reuse_slot[0], self.scale, self.d, self.ws, self.ws_bytes)
        K.kvb_topk(c, sh, ds, B, N, self.cu_tok, self.d, self.k_cap_d, self.ranking, self.s_count, self.sel[0],
                   self.cu_rows[0], self.cursor, self.ws, self.ws_bytes)
        self.cur = 0
        if hook:
            hook(1, self)
        T = self._read_rows(0) if self.cfg.exact_rows else self.T_sel
        for l in range(2, self.L + 1):
            if T == 0:
                self._pt_reuse_rows.add(l)
                if hook:
                    hook(l, self)
                continue
            self._tier_need(l, self.L)
            self._layer_rows(l, T, self._n_rows_ptr(0), self.sel[0], self.cu_rows[0], None, K.KVB_ALPHA_ONE, None,
                             None, None)
            if hook:
                hook(l, self)

    def _link_static(self, hook):
        c, sh, ds, T = self.ctx, self.sh, self.desc, self.T_sel
        if T == 0:
            return
        K.kvb_embed(c, sh, ds, T, None, self.lego_sel, self.tok_l, self.shape.vocab, self.model.embedding,
                    self.hidden)
        for l in range(1, self.L + 1):
            self._tier_need(l, self.L)
            self._layer_rows(l, T, None, self.lego_sel, self.lego_cu, None, K.KVB_ALPHA_ONE, None, None, None)
            if hook:
                hook(l, self)

    # ------------------------------------------------------------------ page tables
    def final_page_table(self) -> torch.Tensor:
        """[L, N] slot of every token's K/V in each layer after the last link step."""
        for l in sorted(self._pt_reuse_rows):
            K.kvb_slot_map(self.ctx, self.sh, self.desc, self.B, self.N, 0, None, None, self.reuse_slot[l - 1], None,
                           None, self.page_table[l - 1], None)
        self._pt_reuse_rows = set()
        return self.page_table

    # ------------------------------------------------------------------ decode continuation
    def decode_init(self, overwrite_first: bool = True, consume_cache: bool = False, graph: bool = False):
        """Prepare decode steps after a link step (CacheSlide page, SLIDE: decode
        writes its K/V first into the original slots of the tokens recomputed in
        that layer, whose reused K/V the new pages superseded, and only then into
        newly allocated pages).

        graph=True records one decode step (the page-table update and every
        layer's launches) as a HIP graph on its first call and replays it for
        each token; the step's token ids, rows, positions and slots reach the
        graph through fixed device buffers written before each replay.

        Overwriting those slots changes the compile pages, so it needs either the
        host tier (every link step reloads them) or consume_cache=True.  Slots of
        chunk instances shared with other requests are never overwritten.
        overwrite_first=False appends every decode token to new pages."""
        if self.max_decode <= 0:
            raise ValueError("the engine was built with max_decode=0")
        if overwrite_first and self.cfg.reuse_tier != "host" and not consume_cache:
            raise ValueError("overwrite-first decode rewrites the compile pages: use reuse_tier='host' or "
                             "consume_cache=True")
        B, L, md, dev = self.B, self.L, self.max_decode, self.device
        for per_layer in getattr(self, "dec_pages", []):  # pages of an earlier decode run
            for ids in per_layer:
                if ids:
                    K.kvb_pool_release(self.pool, ids)
        pt = self.final_page_table().cpu().numpy()
        self._tier_fill_for_decode(pt)
        cu = self.cu_tok_h
        # decode token space: request b's prompt at dcu[b] .. dcu[b] + N_b, then its max_decode tokens
        self.dec_cu = np.array([cu[b] + b * md for b in range(B)], dtype=np.int64)
        Nd = self.N + B * md
        g_of = np.concatenate([np.arange(cu[b], cu[b + 1]) + b * md for b in range(B)]) if self.N else np.zeros(0)
        pt_dec = np.full((L, Nd), -1, dtype=np.int32)
        pt_dec[:, g_of.astype(np.int64)] = pt
        lo_dec = np.zeros(Nd, dtype=np.int32)
        for b in range(B):
            lo_dec[self.dec_cu[b]:self.dec_cu[b] + self.req_lens[b] + md] = self.dec_cu[b]
        # overwritable slots per (layer, request): reused slots of the tokens the layer recomputed,
        # in token order, on chunk instances this request alone uses
        owners = {}
        for b, r in enumerate(self.requests):
            for c in r.chunks:
                owners.setdefault(c.uid, set()).add(b)
        own = np.zeros(self.N, dtype=bool)
        for b, r in enumerate(self.requests):
            g = cu[b]
            for c in r.chunks:
                own[g:g + len(c.tokens)] = _cached(c) and len(owners[c.uid]) == 1
                g += len(c.tokens)
        self.dec_holes = [[None] * B for _ in range(L + 1)]
        for l in range(1, L + 1):
            moved = (pt[l - 1] != self.reuse_slot_h[l - 1]) & own
            for b in range(B):
                seg = slice(cu[b], cu[b + 1])
                self.dec_holes[l][b] = (self.reuse_slot_h[l - 1][seg][moved[seg]].astype(np.int64).tolist()
                                        if overwrite_first else [])
        self.dec_pages = [[[] for _ in range(B)] for _ in range(L + 1)]
        self.dec_t = 0
        self.dec_overwrite_first = overwrite_first
        self.pt_dec = _i32(pt_dec, dev)
        self.lo_dec = _i32(lo_dec, dev)
        self.dec_slots_h = np.full((L, B, md), -1, dtype=np.int64)  # slot of decode token t per layer, request
        self.hidden_dec = torch.zeros((B, self.shape.d_model), dtype=self.tdtype, device=dev)
        # per-step inputs of a decode step, in fixed buffers (what a recorded graph reads)
        self._dec_tok = torch.zeros(B, dtype=torch.int32, device=dev)
        self._dec_rows = torch.zeros(B, dtype=torch.int32, device=dev)
        self._dec_rows64 = torch.zeros(B, dtype=torch.int64, device=dev)
        self._dec_pos = torch.zeros(B, dtype=torch.int32, device=dev)
        self._dec_slots = torch.zeros((L, B), dtype=torch.int32, device=dev)
        self._dec_graph_on = graph
        self._dec_graph = None

    def _dec_slot(self, l: int, b: int, t: int) -> int:
        holes = self.dec_holes[l][b]
        if t < len(holes):
            return holes[t]
        j = t - len(holes)  # j-th appended token of this layer and request
        pages = self.dec_pages[l][b]
        while len(pages) <= j // PAGE:
            pages.extend(K.kvb_pool_alloc(self.pool, 1))
        return pages[j // PAGE] * PAGE + j % PAGE

    def decode_step(self, tokens) -> torch.Tensor:
        """One decode token per request (vocabulary ids `tokens`, one per request)
        at position N_b + t: embed, then per layer QKV + RoPE, K/V into the slot
        the placement gives, attention over the request's prompt (the link
        step's page table) and earlier decode tokens, O-projection + MLP.
        Returns the new tokens' hidden rows [B, d] after the last layer."""
        B, L, t = self.B, self.L, self.dec_t
        if t >= self.max_decode:
            raise ValueError("max_decode tokens already decoded")
        rows = self.dec_cu + np.array(self.req_lens) + t            # decode-space ids of the new tokens
        slots = np.array([[self._dec_slot(l, b, t) for b in range(B)] for l in range(1, L + 1)], dtype=np.int64)
        self.dec_slots_h[:, :, t] = slots
        with torch.cuda.stream(self.stream):
            self._dec_tok.copy_(torch.as_tensor(np.asarray(tokens, dtype=np.int32)))
            self._dec_rows.copy_(torch.as_tensor(rows.astype(np.int32)))
            self._dec_rows64.copy_(torch.as_tensor(rows.astype(np.int64)))
            self._dec_pos.copy_(torch.as_tensor((np.array(self.req_lens) + t).astype(np.int32)))
            self._dec_slots.copy_(torch.as_tensor(slots.astype(np.int32)))
        if not self._dec_graph_on:
            self._decode_body(self.stream)
        elif self._dec_graph is None:
            # first step: run it, then record it (a step is idempotent: the embedding
            # resets the rows and every write repeats the same values)
            self._decode_body(self.stream)
            self.stream.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._decode_body(torch.cuda.current_stream())
            self._dec_graph = g
        else:
            with torch.cuda.stream(self.stream):
                self._dec_graph.replay()
        self.dec_t = t + 1
        return self.hidden_dec

    def _decode_body(self, stream):
        """The launches of one decode step on `stream`, reading its per-step
        inputs from the fixed decode buffers."""
        B, L = self.B, self.L
        c, ds, m = self.ctx, self.desc, self.model
        sh = K.stream_handle(stream)
        pt = self.pt_dec
        with torch.cuda.stream(stream):
            pt.index_copy_(1, self._dec_rows64, self._dec_slots)
        # every layer's K/V of the new tokens goes to the slots placed for it: their pages are dirty
        K.kvb_page_dirty_add(c, sh, ds, L * B, None, self._dec_slots, self.n_pages, self.page_dirty)
        K.kvb_embed(c, sh, ds, B, None, None, self._dec_tok, self.shape.vocab, m.embedding, self.hidden_dec)
        for l in range(1, L + 1):
            W = m.layers[l - 1]
            K.kvb_qkv_fused(c, sh, ds, B, None, None, self.hidden_dec, W["norm1"], W["w_qkv"], self._dec_pos,
                            self.q, self.k, self.v, self.k_pool, self.v_pool, self.n_pages, None,
                            self._dec_slots[l - 1], K.KVB_ALPHA_ONE, None, None, None, self.ws, self.ws_bytes,
                            K.KVB_QKV_SPLIT_K)
            K.kvb_sparse_query_attn(c, sh, ds, B, None, self._dec_rows, self.lo_dec, self.q, self.k_pool, self.v_pool,
                                    self.n_pages, pt[l - 1], self.scale, self.o, self.ws, self.ws_bytes)
            K.kvb_mlp(c, sh, ds, B, None, None, self.o, W["w_o"], self.hidden_dec, W["norm2"], W["w_gate_up"],
                      W["w_down"], self.ws, self.ws_bytes)

    # ------------------------------------------------------------------ results
    def spill_order(self, pages=None) -> List[int]:
        """Pages in SLIDE's eviction order under memory pressure (clean pages
        first, then dirty pages by their counter, largest first), from the
        device counters (host copy, synchronises).  `pages`: the candidates
        (default: every page of the pool)."""
        counts = self.page_dirty.cpu().numpy()
        return spill_order(counts, range(self.n_pages) if pages is None else pages)

    def selected(self, which: Optional[int] = None) -> List[np.ndarray]:
        """Current S_k per request (host copy, synchronises)."""
        w = self.cur if which is None else which
        cu = self.cu_rows[w].cpu().numpy()
        sel = self.sel[w].cpu().numpy()
        return [sel[cu[b]:cu[b + 1]].copy() for b in range(self.B)]
