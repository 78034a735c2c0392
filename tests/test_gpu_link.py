"""End-to-end parity of the compile and link steps on the GPU against the oracle.

Small workloads (the oracle finishes in seconds):
  * tiny decoder, float32, free-running end to end (CacheSlide, 2 layers);
  * the same shape with 8 layers (so the every-4-layers refresh runs) and a
    bfloat16 stack with the large configs' head geometry, both teacher-forced
    layer by layer: the oracle takes the GPU's inputs to layer l (hidden rows,
    S_k, alpha, cached KV) and computes layer l, so a tolerated near-tie in a
    selection cannot cascade;
  * LegoLink on both shapes;
  * page tables bit-exact, chunk-0 deviation exactly zero, bitwise
    determinism run to run.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import link as OL
from oracle import model as OM
from oracle import pages as OP
from oracle import select as OS
from selective_kv_cache_amd import _lib as K
from selective_kv_cache_amd.link import LinkConfig, LinkEngine, Model
from conftest import oracle_inputs
from helpers import TOL, max_rel_err, np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


RULES = {"literal": K.KVB_REFRESH_LITERAL, "dissim": K.KVB_REFRESH_DISSIM}


def build_engine(w, tau=None, mode=None, rule="literal", tier="hbm", **kw):
    s = w.shape
    E = wl.embedding_table(w, DEV)
    layers = [wl.layer_weights(w, l, DEV) for l in range(1, s.n_layers + 1)]
    cfg = LinkConfig(mode=mode or w.mode, ratio=w.ratio, cb_ratio=w.cb_ratio, tau=w.tau if tau is None else tau,
                     period=w.period, lego_k=w.lego_k, refresh_rule=RULES[rule], reuse_tier=tier)
    eng = LinkEngine(Model(s, E, layers), w.requests, cfg, device=DEV, **kw)
    E_np = np64(E)
    W_cache = {}

    def W(l):
        if l not in W_cache:
            W_cache[l] = {k: np64(v) for k, v in layers[l - 1].items()}
        return W_cache[l]

    return eng, E_np, W


def pool_rows(eng, pool, slots):
    slots = np.asarray(slots, dtype=np.int64)
    idx = torch.as_tensor(slots, device=pool.device)
    return np64(pool[idx // 16, :, idx % 16, :])


class Recorder:
    """Hook that copies the engine's state after each layer and refresh."""

    def __init__(self):
        self.after = {}

    def __call__(self, key, eng):
        torch.cuda.synchronize()
        cur = eng.cur
        cu = eng.cu_rows[cur].cpu().numpy()
        st = dict(hidden=eng.hidden.clone(), alpha=eng.alpha.clone(), cursor=eng.cursor.clone(),
                  sel=eng.sel[cur].clone(), cu_rows=cu.copy(), slot_map=eng.slot_map.clone(),
                  dst=eng.dst_slot.clone(), q=eng.q.clone(), k=eng.k.clone(), v=eng.v.clone(), o=eng.o.clone(),
                  dev=eng.dev_l.clone(), cksim=eng.cksim.clone(), d=eng.d.clone(), ranking=eng.ranking.clone(),
                  s_count=eng.s_count.clone())
        self.after[key] = st


def rows_of(st, b=0):
    cu = st["cu_rows"]
    return st["sel"].cpu().numpy()[cu[b]:cu[b + 1]].astype(np.int64)


def compile_pages(eng):
    """(K, V) page arrays holding the compile step's output: the device pool, or
    its pinned host mirror when the link step loads the reused KV from there."""
    if eng.cfg.reuse_tier == "host":
        return eng.host_k, eng.host_v
    return eng.k_pool, eng.v_pool


def compile_check(eng, w, E, W, compiled):
    """Compile-step KV in the GPU pages vs the oracle's per-chunk prefill."""
    s = w.shape
    kc, vc = compile_pages(eng)
    worst = 0.0
    for c in w.compile_chunks:
        for l in range(1, s.n_layers + 1):
            slots = OP.slot_of(eng.comp_pages[c.uid][l - 1], np.arange(len(c)))
            worst = max(worst, max_rel_err(pool_rows(eng, kc, slots), compiled[c.uid][0][l - 1]))
            worst = max(worst, max_rel_err(pool_rows(eng, vc, slots), compiled[c.uid][1][l - 1]))
    return worst


def tie_band_ok(d_ref, S_gpu, S_ref, k):
    """Selections may differ only by tokens whose deviation lies within 1e-3
    (relative) of the k-th largest."""
    diff = set(S_gpu) ^ set(S_ref)
    if not diff:
        return diff
    kth = sorted(d_ref, reverse=True)[k - 1]
    assert all(abs(d_ref[i] - kth) <= 1e-3 * kth for i in diff), "selection differs outside the tie band"
    return diff


def page_plan_check(eng, w):
    """Library page plan == oracle allocator plan, bit for bit."""
    s = w.shape
    alloc = OP.PageAllocator(eng.n_pages)
    plan = OP.compile_plan(w.compile_chunks, s.n_layers, alloc)
    for uid, pages in plan.items():
        assert eng.comp_pages[uid] == pages
    for b, r in enumerate(w.requests):
        lego_rows = OL.legolink_rows(r, w.lego_k).size
        for l in range(1, s.n_layers + 1):
            ratio = w.cb_ratio if eng.cfg.mode == "cacheblend" else w.ratio
            n = OP.capacity(eng.cfg.mode, r.n_tokens, ratio, lego_rows, l)
            assert eng.link_pages[b][l] == alloc.alloc(OP.n_pages_for(n))
    return plan


def test_tiny_cacheslide_free_running():
    """Tiny decoder, float32, 2 layers, CacheSlide at 26%: end to end vs the oracle.
    If the layer-1 selections differ (only inside the tie band), the oracle
    continues from the GPU's set, so layer 2 is always checked."""
    w = wl.tiny()
    eng, E, W = build_engine(w)
    rec = Recorder()
    eng.run_compile()
    eng.run_link(hook=rec)
    torch.cuda.synchronize()
    s, req = w.shape, w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, s, E, W)
    assert compile_check(eng, w, E, W, compiled) < TOL["fp32"]
    plan = page_plan_check(eng, w)
    k_cap = int(math.floor(w.ratio * req.n_tokens))
    K1, _ = OL.splice(req, compiled, 1)
    st, out1 = OL.wca_layer1(req, s, E, W(1), K1, k_cap)
    g1 = rec.after[1]
    # layer 1: deviation, chunk 0 exactly zero, selection within the tie band
    d_gpu = np64(g1["d"])
    assert np.all(d_gpu[: len(req.chunks[0])] == 0.0)
    assert np.allclose(d_gpu, out1["d"], rtol=1e-4, atol=1e-7)
    S_gpu = rows_of(g1)
    assert len(S_gpu) == k_cap == len(out1["S_k"])
    tie_band_ok(out1["d"], S_gpu.tolist(), out1["S_k"], k_cap)
    assert max_rel_err(g1["hidden"], out1["h"]) < TOL["fp32"]
    # layer 2 (the last), from the GPU's set: logical KV, slot map and final hidden rows
    st.S_k = [int(i) for i in S_gpu]
    Kl, Vl = OL.splice(req, compiled, 2)
    o2 = OL.wca_layer(st, 2, s, W(2), Kl, Vl, gate=2 in OL.refresh_layers(s.n_layers, w.period), tau=w.tau)
    g2 = rec.after[2]
    S = np.asarray(o2["S"])
    assert np.array_equal(rows_of(g2), S)
    sm_ref = OP.slot_map(OP.reuse_slots(req, plan, 2), S, eng.link_pages[0][2])
    assert np.array_equal(g2["slot_map"].cpu().numpy(), sm_ref)
    assert max_rel_err(pool_rows(eng, eng.k_pool, sm_ref), o2["K_log"]) < TOL["fp32"]
    assert max_rel_err(pool_rows(eng, eng.v_pool, sm_ref), o2["V_log"]) < TOL["fp32"]
    assert max_rel_err(np64(g2["hidden"])[S], o2["h_rows"]) < TOL["fp32"]
    eng.close()


def teacher_forced_wca(w, tau, tol, tier="hbm", rule="literal"):
    """Run the GPU link once; check every layer against the oracle fed the GPU's inputs.

    With tier="host" the compile pages live in pinned host memory and their
    device copies are zeroed before the step, so the step sees only what it
    loads; the cached rows every check uses come from the host copy (what the
    compile step produced), never from the pool, so a missing load shows."""
    eng, E, W = build_engine(w, tau=tau, tier=tier, rule=rule)
    rec = Recorder()
    eng.run_compile()
    if tier == "host":
        eng.stage_reuse_to_host(evict=True)
        assert int(torch.count_nonzero(eng.k_pool[: eng.n_compile_pages])) == 0
    eng.run_link(hook=rec)
    torch.cuda.synchronize()
    s, req = w.shape, w.requests[0]
    L = s.n_layers
    compiled = OL.compile_chunks(w.compile_chunks, s, E, W)
    assert compile_check(eng, w, E, W, compiled) < tol
    plan = page_plan_check(eng, w)
    tokens, N = req.tokens, req.n_tokens
    # reuse KV as the GPU compiled it (teacher forcing)
    kc, vc = compile_pages(eng)
    reuse = {l: (pool_rows(eng, kc, OP.reuse_slots(req, plan, l)),
                 pool_rows(eng, vc, OP.reuse_slots(req, plan, l))) for l in range(1, L + 1)}
    # the gate ran after exactly the layers of the schedule that still had rows
    gated = sorted(k[1] for k in rec.after if isinstance(k, tuple))
    ran = [l for l in OL.refresh_layers(L, w.period) if len(rows_of(rec.after[l]))]
    assert gated == ran
    # ---- layer 1
    g1 = rec.after[1]
    pos = np.arange(N)
    q, k, v = OM.qkv(OM.store(E[tokens], s.dtype), pos, W(1), s, blocks=OL.chunk_blocks(req))
    assert max_rel_err(g1["q"][:N], q) < tol and max_rel_err(g1["k"][:N], k) < tol
    assert max_rel_err(g1["v"][:N], v) < tol
    K1 = pool_rows(eng, eng.k_pool, g1["slot_map"].cpu().numpy())
    V1 = pool_rows(eng, eng.v_pool, g1["slot_map"].cpu().numpy())
    assert np.array_equal(K1, np64(g1["k"][:N])) and np.array_equal(V1, np64(g1["v"][:N]))
    o = OM.attention_rows_fast(np64(g1["q"][:N]), pos, K1, V1, np.zeros(N, int), s)
    assert max_rel_err(g1["o"][:N], o) < tol
    h2 = OM.post_attention(OM.store(E[tokens], s.dtype), np64(g1["o"][:N]), W(1), s)
    assert max_rel_err(g1["hidden"][:N], h2) < tol
    d_ref = OS.deviation(np64(g1["k"][:N]), reuse[1][0])
    d_gpu = np64(g1["d"])
    assert np.all(d_gpu[: len(req.chunks[0])] == 0.0)
    assert np.allclose(d_gpu, d_ref, rtol=1e-4, atol=1e-7)
    k_cap = int(math.floor(w.ratio * N))
    ranking, S_k, cursor = OS.top_k(d_gpu, k_cap)     # exact on the GPU's own d
    assert list(rows_of(g1)) == S_k
    assert list(g1["ranking"].cpu().numpy()[:len(ranking)]) == ranking
    h_layer1 = np64(g1["hidden"])
    prev = g1
    n_refresh = 0
    cur_state = cursor
    for l in range(2, L + 1):
        gl = rec.after[l]
        S = rows_of(gl)
        assert np.array_equal(S, rows_of(prev))
        T = S.size
        if T == 0:
            continue
        h_in = np64(prev["hidden"])
        Kr, Vr = reuse[l]
        # slot map (bit-exact) and the new-page rows of S_k
        sm_ref = OP.slot_map(OP.reuse_slots(req, plan, l), S, eng.link_pages[0][l])
        assert np.array_equal(gl["slot_map"].cpu().numpy(), sm_ref)
        q, k, v = OM.qkv(h_in[S], S, W(l), s)
        assert max_rel_err(gl["q"][:T], q) < tol and max_rel_err(gl["k"][:T], k) < tol
        assert max_rel_err(gl["v"][:T], v) < tol
        k_rec, v_rec = np64(gl["k"][:T]), np64(gl["v"][:T])
        a_in = np64(prev["alpha"])[S]
        Kb = OM.store(OS.blend(a_in, k_rec, Kr[S]), s.dtype)
        Vb = OM.store(OS.blend(a_in, v_rec, Vr[S]), s.dtype)
        assert max_rel_err(pool_rows(eng, eng.k_pool, sm_ref[S]), Kb) < tol
        assert max_rel_err(pool_rows(eng, eng.v_pool, sm_ref[S]), Vb) < tol
        d_l = OS.deviation(k_rec, Kr[S])
        assert np.allclose(np64(gl["dev"][:T]), d_l, rtol=1e-4, atol=1e-7)
        assert np.allclose(np64(gl["alpha"])[S], OS.alpha_of(d_l, OS.row_sq(Kr[S])), rtol=1e-4, atol=1e-7)
        # the layer's logical KV: the compile step's rows, fused rows from the new pages
        K_log, V_log = Kr.copy(), Vr.copy()
        K_log[S] = pool_rows(eng, eng.k_pool, sm_ref[S])
        V_log[S] = pool_rows(eng, eng.v_pool, sm_ref[S])
        o = OM.attention_rows_fast(np64(gl["q"][:T]), S, K_log, V_log, np.zeros(T, int), s)
        assert max_rel_err(gl["o"][:T], o) < tol
        h_out = OM.post_attention(h_in[S], np64(gl["o"][:T]), W(l), s)
        assert max_rel_err(np64(gl["hidden"])[S], h_out) < tol
        prev = gl
        if ("refresh", l) in rec.after:
            gr = rec.after[("refresh", l)]
            c_gpu = np64(gl["cksim"][:T])
            assert np.allclose(c_gpu, OS.cksim(k_rec, Kr[S]), atol=2e-5)
            S_next, cur_next, retired = OS.refresh(list(S), c_gpu, float(np.float32(tau)),
                                                   ranking, cur_state, rule)
            assert list(rows_of(gr)) == S_next
            assert int(gr["cursor"].cpu()[0]) == cur_next
            # a token joining the set carries its last computed hidden state: none
            # of the layers since layer 1 recomputed it, so its row is layer 1's output
            joined = np.setdiff1d(S_next, S)
            assert np.array_equal(np64(gl["hidden"])[joined], h_layer1[joined])
            n_refresh += len(retired) > 0
            cur_state = cur_next
            prev = dict(gl, sel=gr["sel"], cu_rows=gr["cu_rows"])
    # SLIDE's dirty-page counters: the selected tokens each layer >= 2 routed into each page
    routes = [(rec.after[l]["slot_map"].cpu().numpy(), rows_of(rec.after[l])) for l in range(1, L + 1)]
    assert np.array_equal(eng.page_dirty.cpu().numpy(), OP.dirty_counts(eng.n_pages, routes))
    eng.close()
    return n_refresh


def test_tiny8_cacheslide_teacher_forced():
    w = wl.tiny(n_layers=8)
    # threshold inside the CKSim spread so that both refresh branches run
    assert teacher_forced_wca(w, tau=0.5, tol=TOL["fp32"]) >= 1


def test_small_bf16_cacheslide_teacher_forced():
    w = wl.small_bf16(n_layers=8)
    teacher_forced_wca(w, tau=0.5, tol=TOL["bf16"])


@pytest.mark.parametrize("make,tol", [(lambda: wl.tiny(n_layers=9), TOL["fp32"]),
                                      (lambda: wl.small_bf16(n_layers=9), TOL["bf16"])], ids=["tiny9", "small-bf16-9"])
def test_host_tier_cacheslide_teacher_forced(make, tol):
    """The link step with the reused KV evicted to the host tier, layer by layer
    against the oracle (overlapped loads, two gates)."""
    assert teacher_forced_wca(make(), tau=0.5, tol=tol, tier="host") >= 1


def test_dissim_rule_teacher_forced():
    """The alternative retire rule (CKSim > 1 - tau) with a threshold inside the
    CKSim spread, so that both branches run."""
    teacher_forced_wca(wl.tiny(n_layers=9), tau=0.5, tol=TOL["fp32"], rule="dissim")


@pytest.mark.parametrize("make", [lambda: wl.tiny(n_layers=3, mode="legolink", lens=(96, 40, 130, 20, 64)),
                                  lambda: wl.small_bf16(n_layers=4, mode="legolink"),
                                  lambda: wl.tiny(n_layers=3, mode="legolink", lens=(96, 40, 130), query_len=45),
                                  lambda: wl.small_bf16(n_layers=4, mode="legolink", query_len=77)],
                         ids=["tiny", "small-bf16", "tiny-query", "small-bf16-query"])
def test_legolink_layers(make):
    w = make()
    w.lego_k = 32
    eng, E, W = build_engine(w)
    rec = Recorder()
    eng.run_compile()
    eng.run_link(hook=rec)
    torch.cuda.synchronize()
    s, req = w.shape, w.requests[0]
    tol = TOL[s.dtype]
    compiled = OL.compile_chunks(w.compile_chunks, s, E, W)
    assert compile_check(eng, w, E, W, compiled) < tol
    plan = page_plan_check(eng, w)
    S = OL.legolink_rows(req, 32)
    hS_ref, outs = OL.static_link(req, S, s, E, W, compiled)
    T = S.size
    h_prev = OM.store(E[req.tokens[S]], s.dtype)
    for l in range(1, s.n_layers + 1):
        gl = rec.after[l]
        sm_ref = OP.slot_map(OP.reuse_slots(req, plan, l), S, eng.link_pages[0][l])
        assert np.array_equal(gl["slot_map"].cpu().numpy(), sm_ref)
        q, k, v = OM.qkv(h_prev, S, W(l), s)
        assert max_rel_err(gl["q"][:T], q) < tol and max_rel_err(gl["k"][:T], k) < tol
        K_log = pool_rows(eng, eng.k_pool, sm_ref)
        V_log = pool_rows(eng, eng.v_pool, sm_ref)
        Kr, Vr = OL.splice(req, compiled, l)
        nonsel = np.setdiff1d(np.arange(req.n_tokens), S)
        assert max_rel_err(K_log[nonsel], Kr[nonsel]) < tol
        assert np.array_equal(K_log[S], np64(gl["k"][:T]))
        o = OM.attention_rows_fast(np64(gl["q"][:T]), S, K_log, V_log, np.zeros(T, int), s)
        assert max_rel_err(gl["o"][:T], o) < tol
        h_out = OM.post_attention(h_prev, np64(gl["o"][:T]), W(l), s)
        assert max_rel_err(np64(gl["hidden"])[S], h_out) < tol
        h_prev = np64(gl["hidden"])[S]
    if s.dtype == "fp32":   # free-running end to end as well
        assert max_rel_err(np64(rec.after[s.n_layers]["hidden"])[S], hS_ref) < TOL["fp32"]
    eng.close()


@pytest.mark.parametrize("make", [lambda: wl.tiny(n_layers=3, mode="cacheblend"),
                                  lambda: wl.small_bf16(n_layers=4, mode="cacheblend")],
                         ids=["tiny", "small-bf16"])
def test_cacheblend_teacher_forced(make):
    """CacheBlend-style link: layer 1 (full recompute, attention-map deviation,
    top-k at 15 %) and every later layer against the oracle fed the GPU's
    inputs; the float32 case is also checked free-running end to end."""
    w = make()
    eng, E, W = build_engine(w)
    rec = Recorder()
    eng.run_compile()
    eng.run_link(hook=rec)
    torch.cuda.synchronize()
    s, req = w.shape, w.requests[0]
    tol = TOL[s.dtype]
    N = req.n_tokens
    compiled = OL.compile_chunks(w.compile_chunks, s, E, W)
    assert compile_check(eng, w, E, W, compiled) < tol
    plan = page_plan_check(eng, w)
    reuse = {l: (pool_rows(eng, eng.k_pool, OP.reuse_slots(req, plan, l)),
                 pool_rows(eng, eng.v_pool, OP.reuse_slots(req, plan, l))) for l in range(1, s.n_layers + 1)}
    g1 = rec.after[1]
    pos = np.arange(N)
    q, k, v = OM.qkv(OM.store(E[req.tokens], s.dtype), pos, W(1), s, blocks=OL.chunk_blocks(req))
    assert max_rel_err(g1["q"][:N], q) < tol and max_rel_err(g1["k"][:N], k) < tol
    d_gpu = np64(g1["d"])
    d_ref = OS.attention_map_deviation(np64(g1["q"][:N]), np64(g1["k"][:N]), reuse[1][0], np.zeros(N, int), s)
    assert np.allclose(d_gpu, d_ref, rtol=1e-3, atol=5e-5)
    assert np.all(d_gpu[: len(req.chunks[0])] == 0.0)
    k_cap = int(math.floor(w.cb_ratio * N))
    ranking, S_k, _ = OS.top_k(d_gpu, k_cap)         # exact on the GPU's own scores
    S = rows_of(g1)
    assert list(S) == S_k and len(S) == k_cap
    assert list(g1["ranking"].cpu().numpy()[:len(ranking)]) == ranking
    T = S.size
    h_prev = np64(g1["hidden"])
    for l in range(2, s.n_layers + 1):
        gl = rec.after[l]
        assert np.array_equal(rows_of(gl), S)
        sm_ref = OP.slot_map(OP.reuse_slots(req, plan, l), S, eng.link_pages[0][l])
        assert np.array_equal(gl["slot_map"].cpu().numpy(), sm_ref)
        q, k, v = OM.qkv(h_prev[S], S, W(l), s)
        assert max_rel_err(gl["q"][:T], q) < tol and max_rel_err(gl["k"][:T], k) < tol
        K_log = pool_rows(eng, eng.k_pool, sm_ref)
        V_log = pool_rows(eng, eng.v_pool, sm_ref)
        assert np.array_equal(K_log[S], np64(gl["k"][:T])) and np.array_equal(V_log[S], np64(gl["v"][:T]))
        nonsel = np.setdiff1d(np.arange(N), S)
        assert np.array_equal(K_log[nonsel], reuse[l][0][nonsel])
        o = OM.attention_rows_fast(np64(gl["q"][:T]), S, K_log, V_log, np.zeros(T, int), s)
        assert max_rel_err(gl["o"][:T], o) < tol
        h_out = OM.post_attention(h_prev[S], np64(gl["o"][:T]), W(l), s)
        assert max_rel_err(np64(gl["hidden"])[S], h_out) < tol
        h_prev = np64(gl["hidden"])
    if s.dtype == "fp32":
        st, outs = OL.cacheblend_link(req, s, E, W, compiled, k_cap)
        if st.S_k == list(S):
            assert max_rel_err(np64(eng.hidden)[S], st.h[S]) < TOL["fp32"]
    eng.close()


def test_link_is_deterministic_and_repeatable():
    """Link runs on the same compiled cache give bitwise-identical results, whether the
    refresh runs right after the fusion (no hook) or after the layer (a hook)."""
    w = wl.small_bf16(n_layers=5)
    eng, E, W = build_engine(w, tau=0.5)
    eng.run_compile()
    outs = []
    for hook in (None, None, lambda *_: None):
        eng.run_link(hook=hook)
        torch.cuda.synchronize()
        outs.append((eng.hidden.clone(), eng.k_pool.clone(), eng.v_pool.clone(), eng.selected()[0].copy(),
                     eng.alpha.clone(), eng.d.clone(), eng.ranking.clone()))
    a = outs[0]
    for b in outs[1:]:
        for x, y in zip(a, b):
            if isinstance(x, np.ndarray):
                assert np.array_equal(x, y)
            else:
                assert torch.equal(x, y)
    eng.close()


def test_query_chunk_needs_legolink():
    """A selection that may leave a query token out is refused: it has no cache."""
    w = wl.tiny(n_layers=2, query_len=8)
    with pytest.raises(ValueError):
        build_engine(w)


@pytest.mark.parametrize("exact", [True, False])
def test_single_chunk_selects_nothing(exact):
    """A one-chunk prompt: d == 0 everywhere, S empty, later layers recompute and write nothing."""
    w = wl.tiny(n_layers=5, lens=(200,))
    eng, E, W = build_engine(w)
    eng.cfg.exact_rows = exact
    eng.run_compile()
    after1 = {}

    def hook(key, e):
        if key == 1:
            torch.cuda.synchronize()
            after1.update(hidden=e.hidden.clone(), k=e.k_pool.clone(), v=e.v_pool.clone())

    eng.run_link(hook=hook)
    torch.cuda.synchronize()
    assert torch.all(eng.d == 0) and int(eng.s_count[0]) == 0 and len(eng.selected()[0]) == 0
    assert torch.equal(eng.hidden, after1["hidden"])
    assert torch.equal(eng.k_pool, after1["k"]) and torch.equal(eng.v_pool, after1["v"])
    eng.close()


@pytest.mark.parametrize("exact", [True, False])
def test_few_deviating_tokens_fill_less_than_capacity(exact):
    """A long first chunk (d == 0) and a short second one: |S| < k, so only |S| rows run in layer 2."""
    w = wl.tiny(n_layers=3, lens=(400, 40))
    eng, E, W = build_engine(w)
    eng.cfg.exact_rows = exact
    eng.run_compile()
    rec = Recorder()
    eng.run_link(hook=rec)
    torch.cuda.synchronize()
    n_dev = int((eng.d[:440] > 0).sum())
    S = rows_of(rec.after[1])
    assert len(S) == n_dev < eng.k_cap[0]
    st2 = rec.after[2]
    assert np.array_equal(rows_of(st2), S)
    # the slot map of layer 2 moves exactly the selected tokens to new slots
    moved = np.nonzero(st2["slot_map"].cpu().numpy()[:440] != eng.reuse_slot_h[1][:440])[0]
    assert np.array_equal(moved, S)
    eng.close()
