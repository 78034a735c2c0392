#!/usr/bin/env python3
"""Link-step benchmark on one MI355X.

One step = one whole link step (splice + slot maps, layer-1 full recompute,
deviation + top-k, selective recompute of layers 2..L with fusion, scatter
into new pages, attention and MLP, cosine refreshes) of one batch of the
workload, with weights, the compiled cache and all index arrays already
resident in HBM.  The compile step and the page plan are done before timing.

Prints one JSON line: selected-tokens/s and latency, the roofline of the
dominant kernel (its average launch duration measured with HIP events on the
engine's stream during the timed steps), a per-kernel breakdown, and the CPU
oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
COPY_BYTES = 256 << 20         # copy probe of --profile-only (fp32 multiply by 1, out of place)
DECODE_TOKENS = 8              # decode continuation leg: tokens per request


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mistral7b-cacheslide-8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tier", action="store_true", help="skip the host-tier (reused KV in pinned host memory) leg")
    ap.add_argument("--no-compile", action="store_true", help="skip timing the compile step")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode continuation leg")
    ap.add_argument("--no-cacheblend", action="store_true", help="skip the CacheBlend-style selection leg")
    ap.add_argument("--no-sustained", action="store_true", help="skip the sustained-set leg")
    ap.add_argument("--no-native", action="store_true", help="skip the leg timing the library's own layer loop")
    ap.add_argument("--rule", choices=["literal", "dissim"], default="literal",
                    help="retire rule of the timed step (dissim: the set stays at k on these weights)")
    ap.add_argument("--profile-only", action="store_true", help="warmup + timed steps only (for rocprofv3)")
    return ap.parse_args()


def kernel_work(eng, layer_rows, layer_pos, shape):
    """Algorithmic FLOPs / bytes per kernel for one link step, from the realised rows per layer."""
    s = shape
    d, F, Hq, Hkv, hd = s.d_model, s.ffn, s.n_q_heads, s.n_kv_heads, s.head_dim
    esz = 2 if s.dtype == "bf16" else 4
    w = {k: 0.0 for k in ("gemm_qkv", "gemm_oproj", "gemm_swiglu", "gemm_down", "attention", "blend_scatter",
                          "deviation", "rope", "rope_fuse", "embed")}
    rows_per_layer = []
    for l, (T, pos_lo) in enumerate(zip(layer_rows, layer_pos), start=1):
        rows_per_layer.append(T)
        w["gemm_qkv"] += 2.0 * T * d * (Hq + 2 * Hkv) * hd
        w["gemm_oproj"] += 2.0 * T * Hq * hd * d
        w["gemm_swiglu"] += 2.0 * T * d * 2 * F
        w["gemm_down"] += 2.0 * T * F * d
        w["attention"] += 4.0 * Hq * hd * float(pos_lo)
        w["blend_scatter"] += T * (6.0 * Hkv * hd * esz + 16.0)
        w["rope"] += T * 2.0 * (Hq + Hkv) * hd * esz
        # RoPE + fusion + scatter in one pass (the step's kernel): Q read and
        # written, K and V read, K and V written to the new slots; CacheSlide's
        # layers 2..L also read the cached K and V and alpha, and write d,
        # alpha and CKSim
        blend = l >= 2 and eng.cfg.mode == "cacheslide"  # the other modes replace the cached rows
        w["rope_fuse"] += T * ((2.0 * Hq + 4.0 * Hkv) * hd * esz + ((2.0 * Hkv * hd * esz + 16.0) if blend else 0.0))
    w["deviation"] += eng.N * (2.0 * Hkv * hd * esz + 16.0)
    # the embedding gathers every token's row, except in LegoLink (its static rows only)
    w["embed"] += (eng.T_sel if eng.cfg.mode == "legolink" else eng.N) * 2.0 * d * esz
    return w, rows_per_layer


def record_schedule(eng):
    """Realised rows and summed visible-key counts per layer of one link step
    (deterministic), plus the state after layer 1 (CacheSlide)."""
    import numpy as np
    import torch

    cfg = eng.cfg
    layer_rows, layer_pos, state1 = [], [], {}

    def hook(key, e):
        if isinstance(key, tuple):
            return
        torch.cuda.synchronize()
        if key == 1 and cfg.mode == "cacheslide":
            layer_rows.append(e.N)
            layer_pos.append(float(sum(n * (n + 1) / 2 for n in e.req_lens)))
            cu = e.cu_rows[e.cur].cpu().numpy()
            ns = int(e.s_count[0].item())
            state1.update(hidden=e.hidden.clone(), alpha=e.alpha.clone(), d=e.d.clone(),
                          ranking=e.ranking[:ns].cpu().numpy().copy(),
                          sel=e.sel[e.cur][:cu[-1]].cpu().numpy().copy())
            return
        if cfg.mode == "cacheslide":
            cu = e.cu_rows[e.cur].cpu().numpy()
            sel = e.sel[e.cur][:cu[-1]].cpu().numpy()
        else:
            cu = e.lego_cu.cpu().numpy()
            sel = e.lego_sel[:cu[-1]].cpu().numpy()
        lo = e.lo_l.cpu().numpy()
        layer_rows.append(int(cu[-1]))
        layer_pos.append(float(np.sum(sel - lo[sel] + 1)))

    eng.run_link(hook=hook)
    torch.cuda.synchronize()
    return layer_rows, layer_pos, state1


def kernel_breakdown(eng, args):
    """Per-kernel time of one link step (untimed pass, every launch bracketed by
    HIP events), after warm-up."""
    from selective_kv_cache_amd import _lib as K

    for _ in range(max(args.warmup, 1)):
        eng.run_link()
    K.kvb_timing_enable(eng.ctx, "")
    eng.run_link()
    breakdown = K.kvb_timing_read(eng.ctx)
    K.kvb_timing_enable(eng.ctx, None)
    return breakdown


def per_kernel_rates(breakdown, work):
    per_kernel = {}
    for name, v in breakdown.items():
        b = BOUND.get(name)
        entry = {"ms_per_step": round(v["ms"], 4), "launches": v["count"]}
        if b and work.get(name):
            if b == "mfma":
                a_ = work[name] / (v["ms"] * 1e-3) / 1e12
                entry.update(achieved_tflops=round(a_, 1), frac=round(a_ / PEAK_BF16_TFLOPS, 4))
            else:
                a_ = work[name] / (v["ms"] * 1e-3) / 1e9
                entry.update(achieved_gbs=round(a_, 1), frac=round(a_ / PEAK_HBM_GBS, 4))
        per_kernel[name] = entry
    return per_kernel


def sustained_leg(eng, args, st, s):
    """The same request under the alternative retire rule (CKSim > 1 - tau), with
    which no token retires on these weights: every layer 2..L recomputes the
    full layer-1 selection, the schedule the method keeps when retired tokens
    are refilled from a ranking that does not run out.  Timed like the
    headline step (HIP events on the engine stream), with its own per-kernel
    breakdown and rates."""
    import numpy as np
    import torch

    from selective_kv_cache_amd import _lib as K

    cfg = eng.cfg
    saved = cfg.refresh_rule
    cfg.refresh_rule = K.KVB_REFRESH_DISSIM
    layer_rows, layer_pos, state1 = record_schedule(eng)
    work, rows_per_layer = kernel_work(eng, layer_rows, layer_pos, s)
    breakdown = kernel_breakdown(eng, args)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(st)
        eng.run_link()
        b.record(st)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in ev]
    cfg.refresh_rule = saved
    ms = float(np.mean(step_ms))
    mfma_work = sum(work[k] for k, b in BOUND.items() if b == "mfma")
    n_sel = len(state1["sel"])
    return {"rule": "dissim", "ms_per_step": ms,
            "step_ms_p10_median_p90": [float(np.percentile(step_ms, 10)), float(np.median(step_ms)),
                                       float(np.percentile(step_ms, 90))],
            "selected_tokens_per_s": n_sel / (ms * 1e-3),
            "recomputed_row_layers": int(sum(rows_per_layer)),
            "recomputed_row_layers_per_s": float(sum(rows_per_layer)) / (ms * 1e-3),
            "rows_per_layer": rows_per_layer,
            "algorithmic_mfma_tflop": mfma_work / 1e12,
            "step_mfma_frac": mfma_work / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "kernels": per_kernel_rates(breakdown, work),
            "note": "retire when CKSim > 1 - tau: no token retires on these weights, so every layer recomputes "
                    "the layer-1 selection; same engine, weights and compiled cache as the headline step"}


def native_loop_leg(eng, args, st, n_selected):
    """The same link step queued by the library's C++ layer loop (kvb_link_run):
    no host synchronisation inside the step, every selective layer launched for
    the layer-1 selection's size (the device row counts bound the work).  Timed
    with HIP events on the engine stream, eagerly and as a replayed HIP graph."""
    import numpy as np
    import torch

    from selective_kv_cache_amd import _lib as K

    k = eng.link_desc()

    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    for _ in range(args.warmup):
        eng.run_link_native(k)
    eager = timed(lambda: eng.run_link_native(k))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvb_link_run(eng.ctx, K.stream_handle(torch.cuda.current_stream()), eng.desc, k)

    def replay():
        with torch.cuda.stream(st):
            g.replay()

    replay()
    torch.cuda.synchronize()
    graph = timed(replay)
    del g
    ms_e, ms_g = float(np.mean(eager)), float(np.mean(graph))
    out = {"ms_per_step": ms_e, "ms_per_step_graph": ms_g,
           "selected_tokens_per_s": n_selected / (ms_e * 1e-3),
           "selected_tokens_per_s_graph": n_selected / (ms_g * 1e-3)}
    if eng.cfg.mode == "cacheslide":
        # the sustained schedule (the set stays at k), where every launch size is the true one
        k.refresh_rule = K.KVB_REFRESH_DISSIM
        eng.run_link_native(k)
        out["ms_per_step_sustained"] = float(np.mean(timed(lambda: eng.run_link_native(k))))
        k.refresh_rule = eng.cfg.refresh_rule
        eng.run_link_native(k)
    out["note"] = ("kvb_link_run: one library call per step, every selective layer launched for the layer-1 "
                   "selection's size with device row counts, no host readback; eager and HIP graph replay; "
                   "ms_per_step_sustained under the retire rule that keeps the set at k (compare sustained)")
    return out


BOUND = {"gemm_qkv": "mfma", "gemm_oproj": "mfma", "gemm_swiglu": "mfma", "gemm_down": "mfma", "attention": "mfma",
         "blend_scatter": "hbm", "deviation": "hbm", "rope": "hbm", "rope_fuse": "hbm", "embed": "hbm"}


def cpu_baseline(w, eng, rec_state, step_flops, layers=(2, 3, 4)):
    """Time the oracle as it stands on a bounded sample: the selective layers 2..4
    (the refresh after layer 4 included) over every selected row, free-running
    from the GPU's layer-1 state; scaled to the link step by the step's
    algorithmic FLOPs over the sampled layers'."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import link as OL

    s = w.shape
    st = rec_state
    sel = st["sel"]
    state = OL.WCAState(h=OL.as_f64(st["hidden"]), alpha=OL.as_f64(st["alpha"]), d=OL.as_f64(st["d"]),
                        ranking=[int(x) for x in st["ranking"]], cursor=len(sel), S_k=[int(x) for x in sel])
    d, F, Hq, Hkv, hd = s.d_model, s.ffn, s.n_q_heads, s.n_kv_heads, s.head_dim
    per_row = 2.0 * (d * (Hq + 2 * Hkv) * hd + Hq * hd * d + 3 * d * F)
    t_sum, f_sum = 0.0, 0.0
    for l in layers:
        Wl = {k: OL.as_f64(v) for k, v in wl.layer_weights(w, l, "cuda:0").items()}
        idx = torch.as_tensor(eng.reuse_slot_h[l - 1], device=eng.k_pool.device, dtype=torch.int64)
        Kr = OL.as_f64(eng.k_pool[idx // 16, :, idx % 16, :])
        Vr = OL.as_f64(eng.v_pool[idx // 16, :, idx % 16, :])
        S = np.asarray(state.S_k, dtype=np.int64)
        f_sum += S.size * per_row + 4.0 * Hq * hd * float(np.sum(S + 1))
        t0 = time.perf_counter()
        OL.wca_layer(state, l, s, Wl, Kr, Vr, l in OL.refresh_layers(s.n_layers, w.period), w.tau)
        t_sum += time.perf_counter() - t0
        del Wl, Kr, Vr
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    k = len(sel)
    t_link = t_sum * step_flops / f_sum
    return {"value": k / t_link, "unit": "selected-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"oracle layers {list(layers)} (the refresh after layer 4 included) over the {k} selected "
                       f"rows of the {eng.N}-token request, free-running from the GPU's layer-1 state (float64 "
                       f"numpy, {threads} BLAS threads): {t_sum:.2f} s; link time scaled as T * FLOPs(link step) / "
                       f"FLOPs(sampled layers) = {t_link:.1f} s"),
            "measured_s": t_sum, "extrapolated_link_s": t_link}


def decode_leg(eng, st):
    """Decode continuation after the last link step: DECODE_TOKENS tokens per
    request, each a full pass over every layer at one row per request,
    attending to the link step's page table.  New tokens go to new pages (the
    HBM-resident cache is not overwritten).  The step is recorded as a HIP
    graph on the first token and replayed for the others; the same tokens are
    also timed with eager launches.  HIP events on the engine stream."""
    import numpy as np
    import torch

    toks = np.random.default_rng(11).integers(0, eng.shape.vocab, size=(DECODE_TOKENS, eng.B))
    n = DECODE_TOKENS - 1
    out = {}
    for graph in (True, False):
        eng.decode_init(overwrite_first=False, graph=graph)
        eng.decode_step(toks[0])  # first step: warm-up (and the recording)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(st)
        for t in range(1, DECODE_TOKENS):
            eng.decode_step(toks[t])
        b.record(st)
        torch.cuda.synchronize()
        out["graph" if graph else "eager"] = a.elapsed_time(b) / n
    ms = out["graph"]
    return {"ms_per_decode_step": ms, "tokens_per_s": eng.B / (ms * 1e-3), "ms_per_decode_step_eager": out["eager"],
            "requests": eng.B, "steps_timed": n,
            "note": "one token per request per step after the link step, placed on new pages; HIP graph replays "
                    "(eager launches alongside)"}


def compile_step(eng, args, st, s):
    """The compile step as a second workload: every chunk instance prefilled
    alone from position 0 into its compile pages (QKV for every layer; attention,
    O-projection and MLP for layers 1..L-1).  HIP events on the engine stream."""
    import numpy as np
    import torch

    d, F, Hq, Hkv, hd, L = s.d_model, s.ffn, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_layers
    lens = [len(c.tokens) for c in eng.chunks]
    Nc = int(sum(lens))
    pos_sum = float(sum(n * (n + 1) / 2 for n in lens))   # sum over tokens of (local position + 1)
    flops = (L * 2.0 * Nc * d * (Hq + 2 * Hkv) * hd
             + (L - 1) * (2.0 * Nc * (Hq * hd * d + 3 * d * F) + 4.0 * Hq * hd * pos_sum))
    for _ in range(max(args.warmup, 1)):
        eng.run_compile()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(st)
        eng.run_compile()
        b.record(st)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms_per_step": ms, "tokens_per_s": Nc / (ms * 1e-3), "tokens": Nc, "algorithmic_tflop": flops / 1e12,
            "achieved_tflops": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS if s.dtype == "bf16" else None,
            "note": "compile step (per-chunk prefill from position 0), median of the timed runs"}


def tier_host(eng, args, st, n_selected):
    """The same link step with the reused KV (compile pages) in pinned host
    memory, each layer's pages copied into the pool during the step: overlapped
    with the recompute (copy stream ahead of it) and serially (copy, then the
    layer), plus the copies alone.  Timed with HIP events on the engine stream."""
    import numpy as np
    import torch

    from selective_kv_cache_amd import _lib as K

    cfg = eng.cfg
    saved = (cfg.reuse_tier, cfg.tier_overlap)
    cfg.reuse_tier = "host"
    eng.stage_reuse_to_host()

    def timed(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    res = {}
    for overlap in (True, False):
        cfg.tier_overlap = overlap
        for _ in range(max(args.warmup, 1)):
            eng.run_link()
        res["overlapped" if overlap else "serial"] = timed(eng.run_link, args.steps)
    # bytes one step loads: every layer's reused pages (layer 1 of CacheSlide: keys only)
    page_b = eng.k_pool[0].numel() * eng.k_pool.element_size()
    layers = list(range(1, eng.L + 1))
    nbytes = sum(len(eng.layer_reuse_pages[l]) * page_b * (1 if (l == 1 and cfg.mode != "legolink") else 2)
                 for l in layers)

    def copies_only():
        for l in layers:
            eng._tier_copy(l, eng.sh)

    copy_ms = timed(copies_only, 3)
    cfg.reuse_tier, cfg.tier_overlap = saved
    return {"ms_per_step_overlapped": res["overlapped"], "ms_per_step_serial": res["serial"],
            "selected_tokens_per_s_overlapped": n_selected / (res["overlapped"] * 1e-3),
            "copies_alone_ms": copy_ms, "bytes_if_every_layer_loads": nbytes,
            "h2d_GBps": nbytes / (copy_ms * 1e-3) / 1e9,
            "note": "reused KV in pinned host memory, each layer's pages copied host-to-device during the step "
                    "(layers left with no rows load nothing); median of the timed steps"}


def cold_hbm_leg(eng, s, dev):
    """The HBM-bound row kernels timed cold: before each call a 1 GiB buffer
    refills the 256 MiB MALL and the L2s, so that no operand is cached.  The
    buffer is read ("clean": the caches then hold clean lines, the kernel's
    own bandwidth) or written ("dirty": the kernel's reads also compete with
    the write-back of the dirty lines the fill leaves).  Deviation over all N
    tokens (layer 1, as in the step) and the standalone fusion + scatter over
    the layer-2 rows (alpha, d and CKSim not written, the new-page slots of the
    last step rewritten with the same kind of values)."""
    import numpy as np
    import torch

    from selective_kv_cache_amd import _lib as K

    esz = 2 if s.dtype == "bf16" else 4
    Hkv, hd = s.n_kv_heads, s.head_dim
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    c, sh, ds = eng.ctx, eng.sh, eng.desc
    T = int(eng.k_cap[0]) if eng.B == 1 else eng.T_sel
    calls = {
        "deviation": (lambda: K.kvb_deviation_topk(c, sh, ds, eng.B, eng.N, eng.cu_tok, eng.k, eng.k_pool, eng.n_pages,
                                                   eng.reuse_slot[0], eng.k_cap_d, eng.d, eng.alpha, eng.ranking,
                                                   eng.s_count, eng.sel[0], eng.cu_rows[0], eng.cursor, eng.ws,
                                                   eng.ws_bytes),
                      eng.N * (2.0 * Hkv * hd * esz + 16.0)),
        "blend_scatter": (lambda: K.kvb_blend_scatter(c, sh, ds, T, eng._n_rows_ptr(0), eng.sel[0], eng.k, eng.v,
                                                      eng.k_pool,
                                                      eng.v_pool, eng.n_pages, eng.reuse_slot[1], eng.dst_slot,
                                                      K.KVB_ALPHA_CURRENT, None, None, None),
                          T * (6.0 * Hkv * hd * esz + 16.0)),
    }
    fn0, _ = calls["deviation"]
    fn0()  # the layer-1 selection in sel[0]; then layer 2's slot map and new-page slots for it
    K.kvb_slot_map(c, sh, ds, eng.B, eng.N, T, eng.cu_rows[0], eng.sel[0], eng.reuse_slot[1], eng.new_pages[2],
                   eng.cu_pages[2], eng.page_table[1], eng.dst_slot)
    out = {}
    for name, (fn, nbytes) in calls.items():
        res = {}
        for mode in ("clean", "dirty"):
            ms = []
            for _ in range(6):
                if mode == "clean":
                    flush.sum()
                else:
                    flush.fill_(1.0)
                K.kvb_timing_enable(c, name)
                fn()
                t = K.kvb_timing_read(c)[name]
                K.kvb_timing_enable(c, None)
                ms.append(t["ms"] / t["count"])
            m = float(np.median(ms[1:]))
            res[mode] = {"ms": m, "GBps": nbytes / (m * 1e-3) / 1e9, "frac": nbytes / (m * 1e-3) / 1e9 / PEAK_HBM_GBS}
        out[name] = dict(res["clean"], bytes=nbytes, dirty=res["dirty"])
    del flush
    torch.cuda.synchronize()
    out["note"] = ("cold: 1 GiB read before each call (clean caches; under 'dirty', written instead); median of 5 "
                   "calls after one warm-up")
    return out


def cacheblend_leg(w, model, args, dev):
    """The same request linked with the CacheBlend-style selection (layer 1 in
    full, attention-map deviation, top 15 %, later layers replace the cached
    K/V): its own engine and compile pages on the same weights, timed with HIP
    events on its stream; the attention-map kernel's share with its algorithmic
    FLOPs (both maps of every token over its visible keys)."""
    import numpy as np
    import torch

    from selective_kv_cache_amd import _lib as K
    from selective_kv_cache_amd.link import LinkConfig, LinkEngine

    s = w.shape
    cfg = LinkConfig(mode="cacheblend", cb_ratio=w.cb_ratio)
    eng = LinkEngine(model, w.requests, cfg, device=dev)
    eng.run_compile()
    for _ in range(max(args.warmup, 1)):
        eng.run_link()
    st = eng.stream
    K.kvb_timing_enable(eng.ctx, "attnmap")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(st)
        eng.run_link()
        b.record(st)
    torch.cuda.synchronize()
    t = K.kvb_timing_read(eng.ctx)
    K.kvb_timing_enable(eng.ctx, None)
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    n_sel = len(eng.selected()[0]) if eng.B == 1 else int(eng.cu_rows[0][-1])
    pos_sum = float(sum(n * (n + 1) / 2 for n in eng.req_lens))
    flops = 2 * 2.0 * s.n_q_heads * s.head_dim * pos_sum
    amap = t.get("attnmap", {"ms": float("nan"), "count": 1})
    amap_ms = amap["ms"] / amap["count"]
    tf = flops / (amap_ms * 1e-3) / 1e12
    out = {"ms_per_step": ms, "selected_tokens_per_s": n_sel / (ms * 1e-3), "selected": n_sel,
           "ratio": w.cb_ratio, "attnmap_ms": amap_ms, "attnmap_algorithmic_tflop": flops / 1e12,
           "attnmap_tflops": tf, "attnmap_mfma_frac": tf / PEAK_BF16_TFLOPS if s.dtype == "bf16" else None,
           "note": "CacheBlend-style selection on the same request; median of the timed steps; the attention-map "
                   "kernel computes every score twice (two passes), its rate counts each score once"}
    eng.close()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads as wl
    from selective_kv_cache_amd import _lib as K
    from selective_kv_cache_amd.link import LinkConfig, LinkEngine, Model

    K.load()  # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    w = wl.NAMED[args.workload]()
    s = w.shape
    t_setup = time.perf_counter()
    E = wl.embedding_table(w, dev)
    layers = [wl.layer_weights(w, l, dev) for l in range(1, s.n_layers + 1)]
    cfg = LinkConfig(mode=w.mode, ratio=w.ratio, tau=w.tau, period=w.period, lego_k=w.lego_k,
                     refresh_rule=K.KVB_REFRESH_DISSIM if args.rule == "dissim" else K.KVB_REFRESH_LITERAL)
    eng = LinkEngine(Model(s, E, layers), w.requests, cfg, device=dev, max_decode=DECODE_TOKENS)
    eng.run_compile()
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s: {w.name}, N={eng.N}, pages={eng.n_pages}", file=sys.stderr,
          flush=True)

    layer_rows, layer_pos, state1 = record_schedule(eng)
    work, rows_per_layer = kernel_work(eng, layer_rows, layer_pos, s)
    # selected tokens of the link step: |S_k| chosen at layer 1 (CacheSlide) or the static set (LegoLink)
    n_selected = len(state1["sel"]) if cfg.mode == "cacheslide" else eng.T_sel
    breakdown = kernel_breakdown(eng, args)
    dominant = max(breakdown, key=lambda k: breakdown[k]["ms"])

    # timed steps: HIP events on the engine stream around each step; the dominant
    # kernel's launches are bracketed with events as they run
    st = eng.stream
    torch.cuda.synchronize()
    K.kvb_timing_enable(eng.ctx, dominant)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(st)
        eng.run_link()
        b.record(st)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in ev]
    dom = K.kvb_timing_read(eng.ctx)[dominant]
    K.kvb_timing_enable(eng.ctx, None)
    if args.profile_only:
        # plain copy of known size (read + write COPY_BYTES each): the yardstick
        # that scales the FETCH_SIZE / WRITE_SIZE counters to bytes
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"profile_only": True, "workload": w.name, "ms_per_step": float(np.mean(step_ms)),
                          "dominant": dominant, "dominant_avg_ms": dom["ms"] / dom["count"],
                          "dominant_launches_per_step": dom["count"] / args.steps, "steps": args.steps,
                          "copy_bytes": COPY_BYTES}), flush=True)
        return
    ms = float(np.mean(step_ms))
    dom_avg_ms = dom["ms"] / dom["count"]
    launches_per_step = dom["count"] / args.steps
    dom_work_per_launch = work[dominant] / launches_per_step
    bound = BOUND.get(dominant, "mfma")
    if bound == "mfma":
        achieved = dom_work_per_launch / (dom_avg_ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if s.dtype == "bf16" else PEAK_FP32_TFLOPS
        unit = "TFLOP/s"
    else:
        achieved = dom_work_per_launch / (dom_avg_ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            import hashlib
            t = json.load(open(tfile))
            src = os.path.join(ROOT, "selective_kv_cache_amd", "csrc", t.get("source", ""))
            cur = hashlib.sha256(open(src, "rb").read()).hexdigest() if os.path.exists(src) else None
            if t.get("kernel") == dominant and t.get("workload") == w.name and t.get("source_sha256") == cur:
                traffic = t.get("bytes_per_launch")
        except Exception:
            traffic = None
    per_kernel = per_kernel_rates(breakdown, work)
    B = eng.B
    out = {
        "metric": "link-step selected-tokens/s",
        "value": n_selected / (ms * 1e-3),
        "unit": "selected-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "latency_ms_per_request": ms / B,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "mode": cfg.mode, "requests": B, "n_tokens": eng.N, "n_layers": s.n_layers,
                   "selected": n_selected, "ratio": w.ratio, "tau": w.tau,
                   "recomputed_row_layers": int(sum(rows_per_layer)), "rows_per_layer": rows_per_layer},
        "recomputed_row_layers_per_s": float(sum(rows_per_layer)) / (ms * 1e-3),
        "roofline": {"kernel": dominant, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic, "avg_launch_ms": dom_avg_ms,
                     "work_per_launch": dom_work_per_launch},
        "kernels": per_kernel,
        "step_ms_min_max": [float(np.min(step_ms)), float(np.max(step_ms))],
        "step_ms_p10_median_p90": [float(np.percentile(step_ms, 10)), float(np.median(step_ms)),
                                   float(np.percentile(step_ms, 90))],
    }
    if cfg.mode == "cacheslide" and not args.no_sustained:
        out["sustained"] = sustained_leg(eng, args, st, s)
    if cfg.mode in ("cacheslide", "legolink") and not args.no_native:
        out["native_loop"] = native_loop_leg(eng, args, st, n_selected)
    if not args.no_decode:
        out["decode"] = decode_leg(eng, st)
    if cfg.mode == "cacheslide":
        out["hbm_cold"] = cold_hbm_leg(eng, s, dev)
    if not args.no_compile:
        out["compile_step"] = compile_step(eng, args, st, s)
    if not args.no_tier:
        out["tier_host"] = tier_host(eng, args, st, n_selected)
    if not args.no_cacheblend and cfg.mode == "cacheslide":
        out["cacheblend"] = cacheblend_leg(w, eng.model, args, dev)
    if not args.no_cpu_baseline and cfg.mode == "cacheslide" and eng.B == 1:
        try:
            step_flops = sum(work[k] for k, b in BOUND.items() if b == "mfma")
            out["cpu_baseline"] = cpu_baseline(w, eng, state1, step_flops)
        except Exception as e:  # the GPU figure stands; say why the CPU leg is missing
            out["cpu_baseline"] = {"value": None, "error": repr(e)}
    print(json.dumps(out), flush=True)
    eng.close()


if __name__ == "__main__":
    main()
