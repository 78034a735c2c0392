"""The library's own layer loop (kvb_link_run) against the same steps queued
one by one from Python.

kvb_link_run queues what LinkEngine.run_link queues with exact_rows=False
(CacheSlide, LegoLink and the CacheBlend-style selection)
(every selective layer launched for the layer-1 selection's size, the device
row counts bounding the work), so every output must be bitwise the same:
hidden rows, both K/V pools, page tables, deviation, alpha, per-layer
deviation and cosine similarity, ranking, cursor, the final selection and the
dirty-page counters.  Run-by-run parity of run_link with the oracle is
checked in test_gpu_link.py; this file transfers it to the library's loop.
A HIP graph recorded around one kvb_link_run call replays to the same
values, with the engine's eager work between replays.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from selective_kv_cache_amd import _lib as K
from selective_kv_cache_amd.link import LinkConfig, LinkEngine, Model

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def two_requests(n_layers=9):
    """Two requests sharing their first chunk (compiled once), fp32 tiny decoder."""
    shape = wl.ModelShape(**{**wl.TINY.__dict__, "n_layers": n_layers})
    tok = lambda uid, n: wl.chunk_tokens(0, uid, n)
    r1 = wl.Request([wl.Chunk(0, "fixed", tok(0, 128)), wl.Chunk(1, "dynamic", tok(1, 96)),
                     wl.Chunk(2, "fixed", tok(2, 64))])
    r2 = wl.Request([wl.Chunk(0, "fixed", tok(0, 128)), wl.Chunk(3, "dynamic", tok(3, 160))])
    return wl.Workload("tiny-2req", shape, "cacheslide", [r1, r2])


CASES = {
    "tiny9-literal-lag": (lambda: wl.tiny(n_layers=9), 0.5, K.KVB_REFRESH_LITERAL, K.KVB_ALPHA_LAG),
    "tiny9-2req-dissim-current": (two_requests, 0.12, K.KVB_REFRESH_DISSIM, K.KVB_ALPHA_CURRENT),
    "bf16-5-literal-lag": (lambda: wl.small_bf16(n_layers=5), 0.5, K.KVB_REFRESH_LITERAL, K.KVB_ALPHA_LAG),
    "bf16-9-dissim-one": (lambda: wl.small_bf16(n_layers=9), 0.12, K.KVB_REFRESH_DISSIM, K.KVB_ALPHA_ONE),
    "lego-tiny": (lambda: wl.tiny(n_layers=3, mode="legolink", lens=(96, 40, 130, 20, 64)), 0.12,
                  K.KVB_REFRESH_LITERAL, K.KVB_ALPHA_LAG),
    "lego-bf16-query": (lambda: wl.small_bf16(n_layers=3, mode="legolink", query_len=24), 0.12,
                        K.KVB_REFRESH_LITERAL, K.KVB_ALPHA_LAG),
    "cacheblend-tiny": (lambda: wl.tiny(n_layers=3, mode="cacheblend"), 0.12, K.KVB_REFRESH_LITERAL,
                        K.KVB_ALPHA_LAG),
    "cacheblend-bf16": (lambda: wl.small_bf16(n_layers=3, mode="cacheblend"), 0.12, K.KVB_REFRESH_LITERAL,
                        K.KVB_ALPHA_LAG),
}


def engine(w, tau, rule, alpha_mode, **kw):
    s = w.shape
    E = wl.embedding_table(w, DEV)
    layers = [wl.layer_weights(w, l, DEV) for l in range(1, s.n_layers + 1)]
    cfg = LinkConfig(mode=w.mode, ratio=w.ratio, tau=tau, period=w.period, lego_k=w.lego_k, refresh_rule=rule,
                     alpha_mode=alpha_mode, exact_rows=False)
    return LinkEngine(Model(s, E, layers), w.requests, cfg, device=DEV, **kw)


def state(eng):
    torch.cuda.synchronize()
    if eng.cfg.mode == "legolink":
        # LegoLink writes the hidden rows of its static set, the pools, the
        # page tables and the dirty counters, nothing of the selection state
        out = {name: getattr(eng, name).clone() for name in ("k_pool", "v_pool", "page_table", "page_dirty")}
        out["hidden"] = eng.hidden[eng.lego_sel.long()].clone()
        return out
    names = ("hidden", "k_pool", "v_pool", "page_table", "d", "alpha", "dev_l", "cksim", "ranking", "s_count",
             "cursor", "page_dirty")
    if eng.cfg.mode == "cacheblend":
        # no fusion and no refresh: alpha and the per-row deviation and similarity are not written
        names = tuple(n for n in names if n not in ("alpha", "dev_l", "cksim"))
    out = {name: getattr(eng, name).clone() for name in names}
    out["selected"] = eng.selected()
    return out


def assert_same(a, b):
    for key in a:
        if key == "selected":
            assert len(a[key]) == len(b[key])
            for x, y in zip(a[key], b[key]):
                assert np.array_equal(x, y), key
        else:
            assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("case", list(CASES))
def test_link_run_matches_per_call_loop(case):
    make, tau, rule, alpha_mode = CASES[case]
    eng = engine(make(), tau, rule, alpha_mode)
    eng.run_compile()
    eng.run_link()
    ref = state(eng)
    # clobber what the step writes, so that nothing can pass by being left over
    eng.hidden.fill_(7)
    eng.page_table.fill_(-9)
    eng.page_dirty.fill_(3)
    eng.d.fill_(-1.0)
    eng.cksim.fill_(-1.0)
    eng.run_link_native()
    got = state(eng)
    assert_same(ref, got)
    if eng.cfg.mode != "legolink":
        # rows were recomputed after layer 1
        assert sum(len(x) for x in got["selected"]) > 0
    eng.close()


def test_link_run_graph_replays():
    """One kvb_link_run recorded as a HIP graph replays to the eager result,
    with the engine's own eager work and synchronisation between replays."""
    make, tau, rule, alpha_mode = CASES["bf16-5-literal-lag"]
    stream = torch.cuda.Stream()
    eng = engine(make(), tau, rule, alpha_mode, stream=stream)
    eng.run_compile()
    eng.run_link_native()
    ref = state(eng)
    desc = eng.link_desc()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvb_link_run(eng.ctx, K.stream_handle(torch.cuda.current_stream()), eng.desc, desc)
    for rep in range(3):
        with torch.cuda.stream(eng.stream):
            eng.hidden.fill_(rep + 1)
            eng.page_table.fill_(-5)
            eng.page_dirty.fill_(rep)
        eng.run_link()  # the engine's own eager step in between
        torch.cuda.synchronize()
        with torch.cuda.stream(eng.stream):
            eng.hidden.fill_(rep + 1)
            g.replay()
        got = state(eng)
        assert_same(ref, got)
    eng.close()


def test_link_run_nothing_selected():
    """One chunk: d == 0 everywhere, no row after layer 1; every later layer's
    page table is the reused slots and nothing else changes."""
    w = wl.tiny(n_layers=5, lens=(200,))
    eng = engine(w, 0.12, K.KVB_REFRESH_LITERAL, K.KVB_ALPHA_LAG)
    eng.run_compile()
    eng.run_link()
    eng.final_page_table()
    ref = state(eng)
    eng.page_table.fill_(-9)
    eng.run_link_native()
    got = state(eng)
    assert_same(ref, got)
    assert sum(len(x) for x in got["selected"]) == 0
    eng.close()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("make", [wl.mistral_cacheslide, wl.mistral_legolink, wl.mistral_batch8],
                         ids=["cacheslide-8k", "legolink-16k", "batch8"])
def test_link_run_fullsize(make):
    """At the benchmark sizes (the Mistral-shaped 8192-token CacheSlide request,
    the 16384-token LegoLink prompt and the batch of 8 requests sharing fixed
    chunks; bf16, 32 layers) the library's loop is bitwise the per-call loop
    with device row counts."""
    w = make()
    eng = engine(w, w.tau, K.KVB_REFRESH_LITERAL, K.KVB_ALPHA_LAG)
    eng.run_compile()
    eng.run_link()
    ref = state(eng)
    eng.hidden.fill_(7)
    eng.page_table.fill_(-9)
    eng.page_dirty.fill_(3)
    eng.run_link_native()
    got = state(eng)
    assert_same(ref, got)
    eng.close()
