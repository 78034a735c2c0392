"""Parity at the benchmark configurations' full sizes, on sampled outputs.

The link step runs on the GPU exactly as the benchmark runs it (LinkEngine,
same launches); the oracle cannot redo a whole 8K-32K-token step on the CPU,
so every check is teacher-forced and sampled:

  * integer work in full: the page plan and every checked layer's slot map
    bit-exact, the layer-1 ranking and S_k bit-exact as the top-k of the GPU's
    own deviations, chunk-0 deviations exactly zero, refresh decisions
    bit-exact from the GPU's own CKSim values;
  * floating point on sampled rows: Q/K/V, the fused K/V written to the new
    pages, d and alpha, the attention output and the layer's output hidden
    row, each against the oracle fed the GPU's inputs to that layer (hidden
    rows, alpha, the layer's paged K/V); CKSim of every selected row.

Workloads: the Mistral-7B-shaped 8192-token CacheSlide request (also run
with the CacheBlend-style selection), the 16384-token LegoLink prompt, the
batch of 8 requests with shared fixed chunks, and the Llama-3-70B-shaped
32768-token request (layers 1, 2, 5 and 80).
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import model as OM
from oracle import pages as OP
from oracle import select as OS
from helpers import TOL, max_rel_err, np64
from test_gpu_link import build_engine, page_plan_check, pool_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_SAMPLE = 6


class LayerRecorder:
    """Keeps the engine state after the listed layers (and refreshes) only."""

    def __init__(self, keep):
        self.keep = set(keep)
        self.after = {}

    def __call__(self, key, eng):
        lk = key[1] if isinstance(key, tuple) else key
        if lk not in self.keep:
            return
        torch.cuda.synchronize()
        cur = eng.cur
        self.after[key] = dict(
            hidden=eng.hidden.clone(), alpha=eng.alpha.clone(), cursor=eng.cursor.cpu().numpy().copy(),
            sel=eng.sel[cur].cpu().numpy().copy(), cu_rows=eng.cu_rows[cur].cpu().numpy().copy(),
            slot_map=eng.slot_map.cpu().numpy().copy(), q=eng.q.clone(), k=eng.k.clone(), v=eng.v.clone(),
            o=eng.o.clone(), dev=eng.dev_l.clone(), cksim=eng.cksim.clone(), d=eng.d.clone(),
            ranking=eng.ranking.cpu().numpy().copy(), s_count=eng.s_count.cpu().numpy().copy())


def layer_weights_np(w, l):
    return {k: np64(v) for k, v in wl.layer_weights(w, l, DEV).items()}


def rows_in_order(eng, st):
    """(row index r, global token g, request b) of every recomputed row of a layer state."""
    if st is None:
        return None
    out = []
    for b in range(eng.B):
        for r in range(st["cu_rows"][b], st["cu_rows"][b + 1]):
            out.append((r, int(st["sel"][r]), b))
    return out


def sample_rows(rows, g):
    if len(rows) <= N_SAMPLE:
        return rows
    pick = {0, len(rows) - 1} | set(g.choice(len(rows), N_SAMPLE - 2, replace=False).tolist())
    return [rows[i] for i in sorted(pick)]


def check_rows(eng, w, l, Wl, st, rows, h_in, alpha_in, tol, fused):
    """Q/K/V, fused K/V in the pool, d / alpha, attention and output hidden of sampled rows."""
    s = w.shape
    cu = eng.cu_tok_h
    r_idx = np.array([r for r, _, _ in rows])
    g_idx = np.array([g for _, g, _ in rows])
    b_idx = np.array([b for _, _, b in rows])
    pos = g_idx - cu[b_idx]
    q, k, v = OM.qkv(h_in, pos, Wl, s)
    qg, kg, vg = np64(st["q"][r_idx]), np64(st["k"][r_idx]), np64(st["v"][r_idx])
    assert max_rel_err(qg, q) < tol and max_rel_err(kg, k) < tol and max_rel_err(vg, v) < tol
    sm = st["slot_map"]
    Kr = pool_rows(eng, eng.k_pool, eng.reuse_slot_h[l - 1][g_idx])
    Vr = pool_rows(eng, eng.v_pool, eng.reuse_slot_h[l - 1][g_idx])
    K_new = pool_rows(eng, eng.k_pool, sm[g_idx])
    V_new = pool_rows(eng, eng.v_pool, sm[g_idx])
    if fused:
        # K, V <- a k_rec + (1 - a) k_reuse with the GPU's own k_rec (one rounding)
        assert max_rel_err(K_new, OM.store(OS.blend(alpha_in, kg, Kr), s.dtype)) < tol
        assert max_rel_err(V_new, OM.store(OS.blend(alpha_in, vg, Vr), s.dtype)) < tol
        d_l = OS.deviation(kg, Kr)
        assert np.allclose(np64(st["dev"][r_idx]), d_l, rtol=1e-4, atol=1e-7)
        assert np.allclose(np64(st["alpha"][g_idx]), OS.alpha_of(d_l, OS.row_sq(Kr)), rtol=1e-4, atol=1e-7)
    else:
        assert np.array_equal(K_new, kg) and np.array_equal(V_new, vg)
    # attention of the sampled rows over their request's paged keys of this layer
    og = np64(st["o"][r_idx])
    for b in sorted(set(b_idx.tolist())):
        m = b_idx == b
        last = int(g_idx[m].max())
        keys = np.arange(cu[b], last + 1)
        Kl = np.zeros((last + 1, s.n_kv_heads, s.head_dim))
        Vl = np.zeros_like(Kl)
        Kl[keys] = pool_rows(eng, eng.k_pool, sm[keys])
        Vl[keys] = pool_rows(eng, eng.v_pool, sm[keys])
        o = OM.attention_rows(qg[m], g_idx[m], Kl, Vl, np.full(int(m.sum()), cu[b]), s)
        assert max_rel_err(og[m], o) < tol
    h_out = OM.post_attention(h_in, og, Wl, s)
    assert max_rel_err(np64(st["hidden"][g_idx]), h_out) < tol


def run_fullsize(w, check_layers, seed=0, rule="literal", table_only=()):
    """Link step at full size, then the checks above on the listed layers.

    Every listed layer must recompute rows, except the CacheSlide layers in
    `table_only`: the set has emptied before them, and for those the layer's
    final page table must be the reused slots and its new pages untouched."""
    s = w.shape
    L = s.n_layers
    keep = set(check_layers) | {l - 1 for l in check_layers if l > 1}
    eng, _, _ = build_engine(w, rule=rule)
    rec = LayerRecorder(keep)
    eng.run_compile()
    eng.run_link(hook=rec)
    torch.cuda.synchronize()
    rows_per_layer = ([len(rows_in_order(eng, rec.after[l])) for l in sorted(check_layers) if l > 1]
                      if eng.cfg.mode == "cacheslide" else "static")
    print(f"[{w.name}, {rule}] link step done, checking layers {sorted(check_layers)} "
          f"(rows {rows_per_layer} after layer 1)", flush=True)
    plan = page_plan_check(eng, w)
    E = wl.embedding_table(w, DEV)
    g = np.random.default_rng(seed)
    tol = TOL[s.dtype]
    cu = eng.cu_tok_h
    cacheslide = eng.cfg.mode == "cacheslide"
    for l in sorted(check_layers):
        print(f"[{w.name}] layer {l}", flush=True)
        st = rec.after[l]
        Wl = layer_weights_np(w, l)
        if not cacheslide:
            lego = np.concatenate(eng.lego_rows)
            owner = np.searchsorted(cu, lego, side="right") - 1
            rows = [(r, int(gg), int(b)) for r, (gg, b) in enumerate(zip(lego, owner))]
        elif l == 1:
            rows = [(gg, gg, b) for b in range(eng.B) for gg in range(cu[b], cu[b + 1])]
        else:
            rows = rows_in_order(eng, st)
        if cacheslide and l > 1 and not rows:
            # no row left: the engine skips the layer and writes nothing
            assert l in table_only, f"layer {l} recomputes no row"
            pt = eng.final_page_table()[l - 1].cpu().numpy()
            for b, req in enumerate(w.requests):
                assert np.array_equal(pt[cu[b]:cu[b + 1]], OP.reuse_slots(req, plan, l))
                pages = torch.as_tensor(eng.link_pages[b][l], device=DEV, dtype=torch.int64)
                assert int(torch.count_nonzero(eng.k_pool[pages])) == 0
                assert int(torch.count_nonzero(eng.v_pool[pages])) == 0
            print(f"[{w.name}] layer {l}: no rows, page table and new pages checked", flush=True)
            continue
        assert l not in table_only, f"layer {l} was expected to recompute nothing"
        # slot map of the layer, bit-exact, request by request
        for b, req in enumerate(w.requests):
            S_b = np.array([gg for _, gg, bb in rows if bb == b], dtype=np.int64) - cu[b]
            ref = OP.slot_map(OP.reuse_slots(req, plan, l), S_b, eng.link_pages[b][l])
            assert np.array_equal(st["slot_map"][cu[b]:cu[b + 1]], ref)
        if cacheslide and l == 1:
            d_gpu = np64(st["d"])
            for b, req in enumerate(w.requests):
                seg = slice(cu[b], cu[b + 1])
                assert np.all(d_gpu[seg][: len(req.chunks[0])] == 0.0)
                ranking, S_k, cursor = OS.top_k(d_gpu[seg], eng.k_cap[b])
                assert list(st["ranking"][seg][: len(ranking)] - cu[b]) == ranking  # global token ids
                assert int(st["s_count"][b]) == len(ranking) and int(st["cursor"][b]) == cursor
                assert list(st["sel"][st["cu_rows"][b]:st["cu_rows"][b + 1]] - cu[b]) == S_k
            # layer-1 compile keys of sampled tokens (each depends on its embedding only)
            samp = sample_rows(rows, g)
            gi = np.array([gg for _, gg, _ in samp])
            tok = np.concatenate([np.asarray(r.tokens) for r in w.requests])[gi]
            local = np.array([gg - cu[b] for _, gg, b in samp])
            starts = [np.asarray(w.requests[b].chunk_starts) for _, _, b in samp]
            cpos = np.array([lp - st_[np.searchsorted(st_, lp, side="right") - 1] for lp, st_ in zip(local, starts)])
            h0 = OM.store(np64(E[torch.as_tensor(tok, device=DEV).long()]), s.dtype)
            _, kc, vc = OM.qkv(h0, cpos, Wl, s)
            assert max_rel_err(pool_rows(eng, eng.k_pool, eng.reuse_slot_h[0][gi]), kc) < tol
            assert max_rel_err(pool_rows(eng, eng.v_pool, eng.reuse_slot_h[0][gi]), vc) < tol
            kg = np64(st["k"][gi])
            Kr = pool_rows(eng, eng.k_pool, eng.reuse_slot_h[0][gi])
            assert np.allclose(d_gpu[gi], OS.deviation(kg, Kr), rtol=1e-4, atol=1e-7)
            check_rows(eng, w, l, Wl, st, samp, h0, None, tol, fused=False)
            continue
        if not rows:
            continue
        samp = sample_rows(rows, g)
        gi = np.array([gg for _, gg, _ in samp])
        if l == 1:  # LegoLink layer 1: the embeddings of the static rows
            tok = np.concatenate([np.asarray(r.tokens) for r in w.requests])[gi]
            h_in = OM.store(np64(E[torch.as_tensor(tok, device=DEV).long()]), s.dtype)
            alpha_in = None
        else:
            prev = rec.after[("refresh", l - 1)] if ("refresh", l - 1) in rec.after else rec.after[l - 1]
            src = rec.after[l - 1]
            if cacheslide:
                assert np.array_equal(st["sel"][: st["cu_rows"][-1]], prev["sel"][: prev["cu_rows"][-1]])
            h_in = np64(src["hidden"][gi])
            alpha_in = np64(src["alpha"][gi]) if cacheslide else None
        check_rows(eng, w, l, Wl, st, samp, h_in, alpha_in, tol, fused=cacheslide and l > 1)
        if cacheslide and ("refresh", l) in rec.after:
            gr = rec.after[("refresh", l)]
            rr = np.array([r for r, _, _ in rows])
            ga = np.array([gg for _, gg, _ in rows])
            c_gpu = np64(st["cksim"][rr])
            Kr = pool_rows(eng, eng.k_pool, eng.reuse_slot_h[l - 1][ga])
            assert np.allclose(c_gpu, OS.cksim(np64(st["k"][rr]), Kr), atol=2e-5)
            for b in range(eng.B):
                m = np.array([bb == b for _, _, bb in rows])
                seg = slice(cu[b], cu[b + 1])
                S_b = list(ga[m] - cu[b])
                ranking = list(st["ranking"][seg][: int(st["s_count"][b])] - cu[b])
                S_next, cur_next, _ = OS.refresh(S_b, c_gpu[m], float(np.float32(w.tau)), ranking,
                                                 int(st["cursor"][b]), rule)
                assert list(gr["sel"][gr["cu_rows"][b]:gr["cu_rows"][b + 1]] - cu[b]) == S_next
                assert int(gr["cursor"][b]) == cur_next
        del Wl
    eng.close()


@pytest.mark.timeout(300)
def test_mistral_cacheslide_8k_fullsize():
    run_fullsize(wl.mistral_cacheslide(), check_layers=[1, 2, 4, 5, 12, 13])


@pytest.mark.timeout(300)
def test_mistral_cacheslide_8k_sustained_fullsize():
    """The 8192-token request under the alternative retire rule (CKSim > 1 - tau):
    on these weights no token retires, so all 2129 rows run in every layer up
    to 32 (the schedule the sustained benchmark leg times)."""
    run_fullsize(wl.mistral_cacheslide(), check_layers=[2, 16, 17, 32], rule="dissim")


@pytest.mark.timeout(300)
def test_mistral_legolink_16k_fullsize():
    run_fullsize(wl.mistral_legolink(), check_layers=[1, 2, 32])


@pytest.mark.timeout(300)
def test_mistral_legolink_16k_query_fullsize():
    """The 16K LegoLink prompt followed by a 300-token uncached query, which is
    recomputed in every layer (its slots come only from the new pages)."""
    run_fullsize(wl.mistral_legolink(query_len=300), check_layers=[1, 2, 32])


@pytest.mark.timeout(300)
def test_mistral_batch8_fullsize():
    run_fullsize(wl.mistral_batch8(), check_layers=[1, 2, 4, 5])


@pytest.mark.timeout(300)
def test_mistral_cacheblend_8k_fullsize():
    """The CacheBlend-style selection on the 8192-token Mistral-shaped request:
    layer-1 attention-map deviations (chunk 0 exactly zero, sampled tokens
    against the oracle), ranking and S_k bit-exact from the GPU's own scores,
    slot maps and sampled rows of layers 2 and 32 (replace, no fusion)."""
    w = wl.mistral_cacheslide()
    s = w.shape
    eng, _, _ = build_engine(w, mode="cacheblend")
    rec = LayerRecorder({1, 2, 31, 32})
    eng.run_compile()
    eng.run_link(hook=rec)
    torch.cuda.synchronize()
    print(f"[{w.name} cacheblend] link step done", flush=True)
    plan = page_plan_check(eng, w)
    req, N, tol = w.requests[0], eng.N, TOL[s.dtype]
    g = np.random.default_rng(3)
    st = rec.after[1]
    d_gpu = np64(st["d"])
    assert np.all(d_gpu[: len(req.chunks[0])] == 0.0)
    ranking, S_k, cursor = OS.top_k(d_gpu, eng.k_cap[0])
    assert len(S_k) == eng.k_cap[0] == int(math.floor(w.cb_ratio * N))
    assert list(st["ranking"][: len(ranking)]) == ranking and int(st["s_count"][0]) == len(ranking)
    assert list(st["sel"][st["cu_rows"][0]:st["cu_rows"][1]]) == S_k
    assert np.array_equal(st["slot_map"][:N], OP.slot_map(OP.reuse_slots(req, plan, 1), np.arange(N),
                                                          eng.link_pages[0][1]))
    samp = sorted({N - 1, len(req.chunks[0]), len(req.chunks[0]) - 1} | set(g.choice(N, N_SAMPLE).tolist()))
    K_old = pool_rows(eng, eng.k_pool, eng.reuse_slot_h[0][:N])
    ref = OS.attention_map_deviation(np64(st["q"][:N]), np64(st["k"][:N]), K_old, np.zeros(N, int), s, rows=samp)
    assert np.allclose(d_gpu[samp], ref, rtol=1e-3, atol=5e-5)
    for l in (2, 32):
        print(f"[{w.name} cacheblend] layer {l}", flush=True)
        stl = rec.after[l]
        rows = rows_in_order(eng, stl)
        assert [gg for _, gg, _ in rows] == S_k
        ref_sm = OP.slot_map(OP.reuse_slots(req, plan, l), np.asarray(S_k), eng.link_pages[0][l])
        assert np.array_equal(stl["slot_map"][:N], ref_sm)
        samp_r = sample_rows(rows, g)
        gi = np.array([gg for _, gg, _ in samp_r])
        h_in = np64(rec.after[l - 1]["hidden"][gi])
        check_rows(eng, w, l, layer_weights_np(w, l), stl, samp_r, h_in, None, tol, fused=False)
    eng.close()


@pytest.mark.timeout(600)
def test_llama70_cacheslide_32k_fullsize():
    """Layers 1, 2 and 5 in full; under the literal rule the set has emptied long
    before layer 80, whose page table and new pages are checked."""
    run_fullsize(wl.llama70_cacheslide(), check_layers=[1, 2, 5, 80], table_only=(80,))


@pytest.mark.timeout(600)
def test_llama70_cacheslide_32k_sustained_fullsize():
    """The Llama-3-70B-shaped request under the alternative retire rule: all
    8519 rows run in every layer, checked at layers 2, 17, 40 (a gate) and 80."""
    run_fullsize(wl.llama70_cacheslide(), check_layers=[2, 17, 40, 80], rule="dissim")
