"""Decode continuation after the link step (CacheSlide page, SLIDE decode policy).

A decode token of request b at layer l writes its K/V first into the reused
slot of a token recomputed at layer l (superseded by its new page), in token
order and only on chunk instances b alone uses, and then into new pages.
Checked here:

  * placement, bit-exact: the overwritten slots are exactly those, in that
    order; appended tokens fill fresh pages slot by slot; the prompt's page
    table entries are the link step's final page table;
  * the decode tokens' hidden state after the last layer against the oracle,
    which takes the prompt's K/V from the pool through that page table (the
    link step's output) and computes each decode token from its embedding;
  * with the host tier the compile pages are restored by the next link step,
    which is bitwise the same as the first.
"""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402
from oracle import link as OL  # noqa: E402
from oracle import model as OM  # noqa: E402
from oracle import pages as OP  # noqa: E402
from selective_kv_cache_amd.link import LinkConfig, LinkEngine, Model  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def np64(t):
    return OL.as_f64(t)


def shared_pair(seed=0):
    """Two requests sharing their first (fixed) chunk, tiny fp32 decoder, 2 layers."""
    ch = lambda uid, kind, n: wl.Chunk(uid=uid, kind=kind, tokens=wl.chunk_tokens(seed, uid, n))
    fixed = ch(0, "fixed", 96)
    reqs = [wl.Request([fixed, ch(1, "dynamic", 112)]), wl.Request([fixed, ch(2, "dynamic", 80), ch(3, "fixed", 64)])]
    shape = wl.ModelShape(**{**wl.TINY.__dict__, "n_layers": 2})
    return wl.Workload("tiny-shared-pair", shape, "cacheslide", reqs, seed=seed)


def engine(w, tier, n_dec, mode=None, tau=None):
    s = w.shape
    E = wl.embedding_table(w, DEV)
    layers = [wl.layer_weights(w, l, DEV) for l in range(1, s.n_layers + 1)]
    cfg = LinkConfig(mode=mode or w.mode, ratio=w.ratio, tau=w.tau if tau is None else tau, period=w.period,
                     lego_k=w.lego_k, reuse_tier=tier)
    return LinkEngine(Model(s, E, layers), w.requests, cfg, device=DEV, max_decode=n_dec), E, layers


def pool_rows(eng, pool, slots):
    idx = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=pool.device)
    return np64(pool[idx // 16, :, idx % 16, :])


def expected_holes(eng, pt, l, b):
    owners = {}
    for r_i, r in enumerate(eng.requests):
        for c in r.chunks:
            owners.setdefault(c.uid, set()).add(r_i)
    out, g = [], int(eng.cu_tok_h[b])
    for c in eng.requests[b].chunks:
        for j in range(len(c.tokens)):
            if c.cached and len(owners[c.uid]) == 1 and pt[l - 1][g + j] != eng.reuse_slot_h[l - 1][g + j]:
                out.append(int(eng.reuse_slot_h[l - 1][g + j]))
        g += len(c.tokens)
    return out


def check_decode(eng, E, layers, pt, toks, hs, overwrite_first, compiled=None):
    """compiled: the oracle's compile-step K/V per chunk uid.  When given, a prompt
    token whose page-table entry is its reused slot is read from there instead of
    from the pool (so a reused page that was never loaded back shows)."""
    s = eng.shape
    L, B = s.n_layers, eng.B
    n_before = eng.n_compile_pages + sum(len(p) for req in eng.link_pages for p in req[1:])
    pt_dec = eng.pt_dec.cpu().numpy()
    for b in range(B):
        prompt = np.arange(eng.dec_cu[b], eng.dec_cu[b] + eng.req_lens[b])
        assert np.array_equal(pt_dec[:, prompt], pt[:, eng.cu_tok_h[b]:eng.cu_tok_h[b + 1]])
    n_dec = len(toks)
    for l in range(1, L + 1):
        for b in range(B):
            holes = expected_holes(eng, pt, l, b) if overwrite_first else []
            slots = eng.dec_slots_h[l - 1, b, :n_dec]
            k = min(len(holes), n_dec)
            assert list(slots[:k]) == holes[:k]
            app = slots[k:]
            if len(app):
                # appended tokens fill fresh pages (after every compile and link page) slot by slot
                j = np.arange(len(app))
                assert np.all(app // 16 >= n_before) and np.array_equal(app % 16, j % 16)
                pages = app[j % 16 == 0] // 16
                assert len(set(pages.tolist())) == len(pages) and np.array_equal(app // 16, pages[j // 16])
            rows = eng.dec_cu[b] + eng.req_lens[b] + np.arange(n_dec)
            assert np.array_equal(pt_dec[l - 1, rows], slots)
    # SLIDE's dirty-page counters: the link step's selected tokens (layers >= 2, read
    # off the page table) and every decode token's K/V write
    routes = []
    for l in range(1, L + 1):
        S = np.flatnonzero(pt[l - 1] != eng.reuse_slot_h[l - 1])
        routes.append((pt[l - 1], S))
    want = OP.dirty_counts(eng.n_pages, routes, eng.dec_slots_h[:, :, :n_dec].reshape(-1))
    assert np.array_equal(eng.page_dirty.cpu().numpy(), want)
    # hidden state of every decode token after the last layer vs the oracle
    E64 = np64(E)
    W = [{kk: np64(vv) for kk, vv in layers[l].items()} for l in range(L)]
    tol = TOL[s.dtype]
    for b in range(B):
        Nb = eng.req_lens[b]
        for t in range(n_dec):
            h = OM.store(E64[[int(toks[t][b])]], s.dtype)
            for l in range(1, L + 1):
                q, kk, vv = OM.qkv(h, np.array([Nb + t]), W[l - 1], s)
                keys = np.concatenate([pt[l - 1][eng.cu_tok_h[b]:eng.cu_tok_h[b + 1]],
                                       eng.dec_slots_h[l - 1, b, :t]]).astype(np.int64)
                Kp, Vp = pool_rows(eng, eng.k_pool, keys), pool_rows(eng, eng.v_pool, keys)
                if compiled is not None:
                    seg = slice(eng.cu_tok_h[b], eng.cu_tok_h[b + 1])
                    reused = pt[l - 1][seg] == eng.reuse_slot_h[l - 1][seg]
                    Kc, Vc = OL.splice(eng.requests[b], compiled, l, s)
                    Kp[:Nb][reused], Vp[:Nb][reused] = Kc[reused], Vc[reused]
                Kl = np.concatenate([Kp, kk])
                Vl = np.concatenate([Vp, vv])
                o = OM.attention_rows(q, np.array([Nb + t]), Kl, Vl, np.array([0]), s)
                h = OM.post_attention(h, o, W[l - 1], s)
            got = np64(hs[t][b:b + 1])
            err = np.max(np.abs(got - h)) / np.max(np.abs(h))
            assert err < tol, (b, t, err)


def run(w, tier, overwrite_first, n_dec, consume=False, mode=None, evict=False, tau=None):
    eng, E, layers = engine(w, tier, n_dec, mode, tau)
    eng.run_compile()
    if tier == "host":
        eng.stage_reuse_to_host(evict=evict)
    eng.run_link()
    pt = eng.final_page_table().cpu().numpy().copy()
    first = dict(hidden=eng.hidden.clone(), k=eng.k_pool[eng.n_compile_pages:].clone())
    eng.decode_init(overwrite_first=overwrite_first, consume_cache=consume)
    g = np.random.default_rng(7)
    toks = g.integers(0, w.shape.vocab, size=(n_dec, eng.B))
    hs = []
    for t in range(n_dec):
        hs.append(eng.decode_step(toks[t]).clone())
    torch.cuda.synchronize()
    return eng, E, layers, pt, toks, hs, first


@pytest.mark.parametrize("overwrite_first", [True, False])
def test_decode_tiny_host_tier(overwrite_first):
    w = wl.tiny(n_layers=2)
    eng, E, layers, pt, toks, hs, first = run(w, "host", overwrite_first, n_dec=20)
    check_decode(eng, E, layers, pt, toks, hs, overwrite_first)
    # the next link step reloads the compile pages: bitwise the first link step
    eng.run_link()
    torch.cuda.synchronize()
    assert torch.equal(eng.hidden, first["hidden"])
    eng.close()


@pytest.mark.parametrize("overwrite_first", [True, False])
def test_decode_after_evicted_host_tier(overwrite_first):
    """Reused KV evicted to the host tier, and a set that empties at the first gate
    (every token retires, the ranking is exhausted): layers 5-8 run no row, so
    the link step loads none of their reused pages.  Decode must still attend
    over the compile step's K/V there; the reference reads those rows from the
    oracle's compile step, not from the pool."""
    w = wl.tiny(n_layers=8, lens=(400, 40))
    eng, E, layers, pt, toks, hs, first = run(w, "host", overwrite_first, n_dec=6, evict=True, tau=1.5)
    skipped = [l for l in range(1, 9) if np.array_equal(pt[l - 1], eng.reuse_slot_h[l - 1])]
    assert skipped == [5, 6, 7, 8]
    E64 = np64(E)
    W = {l: {kk: np64(vv) for kk, vv in layers[l - 1].items()} for l in range(1, 9)}
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E64, W.__getitem__)
    check_decode(eng, E, layers, pt, toks, hs, overwrite_first, compiled=compiled)
    eng.close()


def test_decode_shared_chunk_never_overwritten():
    w = shared_pair()
    eng, E, layers, pt, toks, hs, first = run(w, "host", True, n_dec=5)
    check_decode(eng, E, layers, pt, toks, hs, True)
    shared = set()
    for l in range(1, w.shape.n_layers + 1):
        for p in eng.comp_pages[0][l - 1]:
            shared.update(range(p * 16, p * 16 + 16))
    assert not shared & set(eng.dec_slots_h.reshape(-1).tolist())
    eng.close()


def test_decode_bf16_legolink_consumes_cache():
    w = wl.small_bf16(n_layers=4, mode="legolink")
    eng, E, layers, pt, toks, hs, first = run(w, "hbm", True, n_dec=3, consume=True)
    check_decode(eng, E, layers, pt, toks, hs, True)
    eng.close()


def test_decode_legolink_query_suffix_has_no_slot_to_overwrite():
    """An uncached query has no reused slot: decode overwrites only the
    superseded slots of recomputed cached tokens, then appends."""
    w = wl.tiny(n_layers=2, mode="legolink", lens=(96, 40, 70), query_len=24)
    n_dec = 80   # more than the cached tokens LegoLink recomputes (32 + 32): some are appended
    eng, E, layers, pt, toks, hs, first = run(w, "host", True, n_dec=n_dec)
    check_decode(eng, E, layers, pt, toks, hs, True)
    assert np.all(eng.dec_slots_h >= 0)
    for l in range(1, w.shape.n_layers + 1):
        assert len(eng.dec_holes[l][0]) == 64
    eng.close()


def test_decode_graph_replays_match_eager():
    """A decode step recorded as a HIP graph and replayed for later tokens gives
    the eager steps' hidden rows and placement bit for bit, replay after replay
    (host work and synchronisations between the replays)."""
    w = wl.small_bf16(n_layers=3)
    n_dec = 6
    eng, E, layers = engine(w, "hbm", n_dec)
    eng.run_compile()
    toks = np.random.default_rng(3).integers(0, w.shape.vocab, size=(n_dec, eng.B))
    runs = []
    for graph in (False, True):
        eng.run_link()
        eng.decode_init(overwrite_first=False, graph=graph)
        hs = []
        for t in range(n_dec):
            hs.append(eng.decode_step(toks[t]).clone())
            torch.cuda.synchronize()
            hs[-1] = hs[-1].cpu()
        runs.append((hs, eng.dec_slots_h.copy(), eng.pt_dec.cpu().clone(), eng.page_dirty.cpu().clone()))
    (h0, s0, p0, c0), (h1, s1, p1, c1) = runs
    assert np.array_equal(s0, s1) and torch.equal(p0, p1) and torch.equal(c0, c1)
    for t in range(n_dec):
        assert torch.equal(h0[t], h1[t]), t
    eng.close()


def test_decode_overwrite_needs_a_reloadable_cache():
    w = wl.tiny(n_layers=2)
    eng, E, layers = engine(w, "hbm", 2)
    eng.run_compile()
    eng.run_link()
    with pytest.raises(ValueError):
        eng.decode_init(overwrite_first=True)
    eng.decode_init(overwrite_first=False)
    eng.close()
