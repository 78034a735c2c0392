"""Pins of the CPU oracle against facts fixed outside it (no GPU).

Each test checks the oracle against something other than itself: a library
routine (torch's RMSNorm / SDPA / complex arithmetic, bfloat16 casts), a closed
form that follows from the pages' definitions, brute force over tiny inputs,
or a hand-worked example under tests/golden/.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as wl
from oracle import link as OL
from oracle import model as OM
from oracle import pages as OP
from oracle import select as OS
from conftest import oracle_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ library reference decoder

def torch_prefill(tokens, shape, E, W, n_layers):
    """Reference decoder built from library routines (float64, CPU):
    F.rms_norm, complex-multiplication RoPE, F.scaled_dot_product_attention
    (causal) with KV heads repeated per group, F.silu."""
    d, hd = shape.d_model, shape.head_dim
    Hq, Hkv = shape.n_q_heads, shape.n_kv_heads
    G = Hq // Hkv
    N = len(tokens)
    h = torch.tensor(E[tokens], dtype=torch.float64)
    pos = torch.arange(N, dtype=torch.float64)
    j = torch.arange(hd // 2, dtype=torch.float64)
    ang = pos[:, None] * torch.pow(torch.tensor(shape.rope_base, dtype=torch.float64), -2.0 * j / hd)[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]          # [N, 1, hd/2]

    def rope_c(x):
        xc = torch.complex(x[..., : hd // 2], x[..., hd // 2:]) * rot
        return torch.cat([xc.real, xc.imag], dim=-1)

    Ks, Vs = [], []
    for l in range(1, n_layers + 1):
        Wl = {k: torch.tensor(v) for k, v in W(l).items()}
        a = F.rms_norm(h, (d,), weight=Wl["norm1"], eps=shape.rms_eps)
        y = a @ Wl["w_qkv"].T
        q = y[:, : Hq * hd].view(N, Hq, hd)
        k = y[:, Hq * hd: (Hq + Hkv) * hd].view(N, Hkv, hd)
        v = y[:, (Hq + Hkv) * hd:].view(N, Hkv, hd)
        q, k = rope_c(q), rope_c(k)
        Ks.append(k.numpy().copy())
        Vs.append(v.numpy().copy())
        o = F.scaled_dot_product_attention(
            q.transpose(0, 1), k.repeat_interleave(G, dim=1).transpose(0, 1),
            v.repeat_interleave(G, dim=1).transpose(0, 1), is_causal=True)
        h = h + o.transpose(0, 1).reshape(N, Hq * hd) @ Wl["w_o"].T
        b = F.rms_norm(h, (d,), weight=Wl["norm2"], eps=shape.rms_eps)
        gu = b @ Wl["w_gate_up"].T
        h = h + (F.silu(gu[:, : shape.ffn]) * gu[:, shape.ffn:]) @ Wl["w_down"].T
    return Ks, Vs, h.numpy()


def tiny64(n_layers=2, **kw):
    return wl.tiny(n_layers=n_layers, dtype="fp64", **kw)


# ------------------------------------------------------------ storage rounding

def test_round_bf16_matches_torch_cast(rng):
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0078125, -1.00390625, 65504.0]])
    ours = OM.round_bf16(x)
    ref = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------ RoPE

def test_rope_properties(rng):
    x = rng.standard_normal((7, 3, 64))
    pos = rng.integers(0, 5000, 7)
    y = OM.rope(x, pos, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.array_equal(OM.rope(x, np.zeros(7, int), 10000.0), x)
    # relative-position property: <R_a q, R_b k> depends on a - b only
    q, k = rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64))
    d1 = (OM.rope(q, [100], 1e4) * OM.rope(k, [37], 1e4)).sum()
    d2 = (OM.rope(q, [1063], 1e4) * OM.rope(k, [1000], 1e4)).sum()
    assert abs(d1 - d2) < 1e-10


def test_rope_matches_complex_rotation(rng):
    x = rng.standard_normal((5, 2, 128))
    pos = np.array([0, 1, 17, 4095, 32767])
    j = np.arange(64)
    z = (x[..., :64] + 1j * x[..., 64:]) * np.exp(1j * pos[:, None, None] * 10000.0 ** (-2 * j / 128))
    ref = np.concatenate([z.real, z.imag], axis=-1)
    assert np.allclose(OM.rope(x, pos, 10000.0), ref, atol=1e-12)


# ------------------------------------------------------------ attention

def test_attention_rows_match_sdpa_and_each_other(rng):
    shape = wl.ModelShape(n_layers=1, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=32, dtype="fp64")
    N = 40
    q = rng.standard_normal((N, 4, 16))
    K = rng.standard_normal((N, 2, 16))
    V = rng.standard_normal((N, 2, 16))
    ref = F.scaled_dot_product_attention(
        torch.tensor(q).transpose(0, 1), torch.tensor(K).repeat_interleave(2, 1).transpose(0, 1),
        torch.tensor(V).repeat_interleave(2, 1).transpose(0, 1), is_causal=True).transpose(0, 1).reshape(N, -1).numpy()
    rows = np.array([0, 3, 4, 17, 39])
    a = OM.attention_rows(q[rows], rows, K, V, np.zeros(5, int), shape)
    b = OM.attention_rows_fast(q[rows], rows, K, V, np.zeros(5, int), shape)
    assert np.allclose(a, ref[rows], atol=1e-12)
    assert np.allclose(b, ref[rows], atol=1e-12)
    # MHA special case (Hq == Hkv) and a lower key bound
    shape1 = wl.ModelShape(n_layers=1, d_model=32, n_q_heads=2, n_kv_heads=2, head_dim=16, ffn=32, dtype="fp64")
    qq = q[:, :2]
    lo = np.array([0, 2, 4, 10, 30])
    c = OM.attention_rows(qq[rows], rows, K, V, lo, shape1)
    for t, r in enumerate(rows):
        for h in range(2):
            s = K[lo[t]:r + 1, h] @ qq[r, h] / 4.0
            p = np.exp(s - s.max())
            assert np.allclose(c[t, h * 16:(h + 1) * 16], (p / p.sum()) @ V[lo[t]:r + 1, h], atol=1e-12)


# ------------------------------------------------------------ full prefill (FR special case)

def test_full_prefill_matches_library_decoder():
    w = tiny64(n_layers=2, lens=(40, 24))
    E, W = oracle_inputs(w)
    toks = w.requests[0].tokens
    K, V, h = OL.full_prefill(toks, w.shape, E, W)
    Kr, Vr, hr = torch_prefill(toks, w.shape, E, W, 2)
    for l in range(2):
        assert np.allclose(K[l], Kr[l], rtol=1e-10, atol=1e-10)
        assert np.allclose(V[l], Vr[l], rtol=1e-10, atol=1e-10)
    assert np.allclose(h, hr, rtol=1e-10, atol=1e-10)


def test_fully_recompute_equals_prefill():
    """EPIC section 3.2 'Fully Recompute': the static link with S = all tokens is
    plain prefill of the spliced prompt (library decoder)."""
    w = tiny64(n_layers=2, lens=(40, 24, 36))
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    hS, _ = OL.static_link(req, np.arange(req.n_tokens), w.shape, E, W, compiled)
    _, _, hr = torch_prefill(req.tokens, w.shape, E, W, 2)
    assert np.allclose(hS, hr, rtol=1e-10, atol=1e-10)


def test_wca_select_all_alpha_one_is_prefill():
    """Selecting every token with alpha forced to 1 reproduces full prefill."""
    w = tiny64(n_layers=3, lens=(40, 24, 36))
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    K1, _ = OL.splice(req, compiled, 1)
    st, _ = OL.wca_layer1(req, w.shape, E, W(1), K1, k_cap=10)
    st.S_k = list(range(req.n_tokens))
    for l in (2, 3):
        Kl, Vl = OL.splice(req, compiled, l)
        OL.wca_layer(st, l, w.shape, W(l), Kl, Vl, gate=False, alpha_mode="one")
    _, _, hr = torch_prefill(req.tokens, w.shape, E, W, 3)
    assert np.allclose(st.h, hr, rtol=1e-10, atol=1e-10)


def test_compile_equals_prefill_of_each_chunk():
    w = tiny64(n_layers=2, lens=(24, 40))
    E, W = oracle_inputs(w)
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    for c in w.compile_chunks:
        Kr, Vr, _ = torch_prefill(c.tokens, w.shape, E, W, 2)
        for l in range(2):
            assert np.allclose(compiled[c.uid][0][l], Kr[l], rtol=1e-10, atol=1e-10)
            assert np.allclose(compiled[c.uid][1][l], Vr[l], rtol=1e-10, atol=1e-10)


# ------------------------------------------------------------ LegoLink with an uncached query suffix

def test_legolink_rows_with_query_worked_example():
    """EPIC section 4: k' = the first k tokens of each chunk (not the first) plus
    the user's query tokens.  Chunks [5, 3, 40] then a 7-token query, k = 4."""
    ch = lambda uid, kind, n: wl.Chunk(uid=uid, kind=kind, tokens=np.zeros(n, dtype=np.int32))
    req = wl.Request([ch(0, "fixed", 5), ch(1, "dynamic", 3), ch(2, "fixed", 40), ch(3, "query", 7)])
    assert OL.legolink_rows(req, 4).tolist() == [5, 6, 7, 8, 9, 10, 11] + list(range(48, 55))
    assert OL.legolink_rows(req, 0).tolist() == list(range(48, 55))
    only_query = wl.Request([ch(9, "query", 6)])
    assert OL.legolink_rows(only_query, 32).tolist() == list(range(6))
    plan = OP.compile_plan([c for c in req.chunks if c.cached], 1, OP.PageAllocator(16))
    assert set(plan) == {0, 1, 2}
    rs = OP.reuse_slots(req, plan, 1)
    assert np.all(rs[48:] == -1) and np.all(rs[:48] >= 0)


def test_legolink_query_after_first_chunk_is_prefill():
    """The first chunk is compiled at positions 0.. already, so its cache is exact;
    a query after it, recomputed in every layer, then matches plain prefill of the
    whole prompt on the query rows (library decoder), and the query's cached rows
    (NaN, there is none) are never read."""
    w = tiny64(n_layers=2, lens=(48,), query_len=20, mode="legolink")
    E, W = oracle_inputs(w)
    req = w.requests[0]
    assert [c.cached for c in req.chunks] == [True, False]
    compiled = OL.compile_chunks(req.chunks, w.shape, E, W)
    assert set(compiled) == {req.chunks[0].uid}
    S = OL.legolink_rows(req, 32)
    assert S.tolist() == list(range(48, 68))
    hS, outs = OL.static_link(req, S, w.shape, E, W, compiled)
    _, _, hr = torch_prefill(req.tokens, w.shape, E, W, 2)
    assert np.all(np.isfinite(hS))
    assert np.allclose(hS, hr[48:], rtol=1e-10, atol=1e-10)
    Kr, _ = OL.splice(req, compiled, 1, w.shape)
    assert np.all(np.isnan(Kr[48:])) and np.all(np.isfinite(outs[0]["K_log"]))


# ------------------------------------------------------------ CacheBlend-style attention-map deviation

def _amd_shape(Hq=4, Hkv=2, hd=16):
    return wl.ModelShape(n_layers=1, d_model=Hq * hd, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=hd, ffn=32,
                         dtype="fp64")


def test_attention_map_deviation_two_keys_closed_form(rng):
    """With two visible keys an attention row is (sigmoid(a), 1 - sigmoid(a)),
    a = (s_0 - s_1); the L1 distance of two such rows is 2 |sigmoid(a) - sigmoid(b)|.
    A token that sees one key has the row (1) under both: deviation 0."""
    from scipy.special import expit
    shape = _amd_shape()
    q = rng.standard_normal((2, 4, 16))
    kn = rng.standard_normal((2, 2, 16))
    ko = rng.standard_normal((2, 2, 16))
    dev = OS.attention_map_deviation(q, kn, ko, np.zeros(2, int), shape)
    assert dev[0] == 0.0
    ref = 0.0
    for h in range(4):
        a = (kn[0, h // 2] - kn[1, h // 2]) @ q[1, h] / 4.0
        b = (ko[0, h // 2] - ko[1, h // 2]) @ q[1, h] / 4.0
        ref += 2.0 * abs(expit(a) - expit(b))
    assert np.isclose(dev[1], ref / 4.0, rtol=1e-12, atol=1e-15)


def test_attention_map_deviation_matches_library_maps(rng):
    """Brute force with library routines: full masked score matrices per head,
    torch.softmax, L1 over each row, mean over heads (GQA 3, per-token key
    lower bounds as in a batch of two requests)."""
    Hq, Hkv, hd, N = 6, 2, 8, 37
    shape = _amd_shape(Hq, Hkv, hd)
    q = rng.standard_normal((N, Hq, hd))
    kn = rng.standard_normal((N, Hkv, hd))
    ko = kn + 0.3 * rng.standard_normal((N, Hkv, hd))
    lo = np.where(np.arange(N) < 20, 0, 20)
    dev = OS.attention_map_deviation(q, kn, ko, lo, shape)
    idx = torch.arange(N)
    allowed = (idx[None, :] <= idx[:, None]) & (idx[None, :] >= torch.as_tensor(lo)[:, None])
    maps = []
    for K in (kn, ko):
        Kr = torch.tensor(K).repeat_interleave(Hq // Hkv, dim=1)                 # [N, Hq, hd]
        S = torch.einsum("ihd,jhd->hij", torch.tensor(q), Kr) / np.sqrt(hd)
        maps.append(torch.softmax(S.masked_fill(~allowed, float("-inf")), dim=-1))
    ref = (maps[0] - maps[1]).abs().sum(-1).mean(0).numpy()
    assert np.allclose(dev, ref, rtol=1e-12, atol=1e-14)


def test_attention_map_deviation_invariants(rng):
    shape = _amd_shape()
    N = 25
    q = rng.standard_normal((N, 4, 16))
    kn = rng.standard_normal((N, 2, 16))
    ko = rng.standard_normal((N, 2, 16))
    lo = np.zeros(N, int)
    dev = OS.attention_map_deviation(q, kn, ko, lo, shape)
    assert np.all(dev >= 0) and np.all(dev <= 2.0)
    assert np.array_equal(OS.attention_map_deviation(q, kn, kn, lo, shape), np.zeros(N))
    assert np.allclose(OS.attention_map_deviation(q, ko, kn, lo, shape), dev, rtol=1e-13)
    # causal: keys after token i do not change its deviation
    ko2 = ko.copy()
    ko2[15:] += 5.0
    dev2 = OS.attention_map_deviation(q, kn, ko2, lo, shape)
    assert np.array_equal(dev2[:15], dev[:15]) and not np.allclose(dev2[15:], dev[15:])
    # identical keys up to token i: zero up to i, whatever follows
    ko3 = kn.copy()
    ko3[10:] = ko[10:]
    assert np.all(OS.attention_map_deviation(q, kn, ko3, lo, shape)[:10] == 0.0)


def test_cacheblend_select_all_is_prefill():
    """Chunk 0 is cached at its own positions, so its tokens' maps agree exactly
    (deviation 0) and they are never selected; selecting every other token and
    replacing its KV in every layer reproduces full prefill (library decoder)."""
    w = tiny64(n_layers=3, lens=(40, 24, 36), mode="cacheblend")
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    st, outs = OL.cacheblend_link(req, w.shape, E, W, compiled, k_cap=req.n_tokens)
    assert np.all(outs[0]["d"][:40] == 0.0) and np.all(outs[0]["d"][40:] > 0.0)
    assert st.S_k == list(range(40, 100))
    _, _, hr = torch_prefill(req.tokens, w.shape, E, W, 3)
    assert np.allclose(st.h[40:], hr[40:], rtol=1e-10, atol=1e-10)
    # a cap below |S| keeps the ranking's top entries, ascending
    st2, outs2 = OL.cacheblend_link(req, w.shape, E, W, compiled, k_cap=9, keep=False)
    d = outs2[0]["d"]
    assert st2.S_k == sorted(sorted(range(100), key=lambda i: (-d[i], i))[:9])


# ------------------------------------------------------------ naive / identical-reuse special cases

def test_naive_link_keeps_cache_bitwise():
    """EPIC section 3.2 'Naive': nothing recomputed, the layer KV is the spliced cache."""
    w = wl.tiny(n_layers=2, lens=(40, 24, 36))
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    assert OL.legolink_rows(req, 0).size == 0
    _, outs = OL.static_link(req, OL.legolink_rows(req, 0), w.shape, E, W, compiled)
    for l in (1, 2):
        K, V = OL.splice(req, compiled, l)
        assert np.array_equal(outs[l - 1]["K_log"], K) and np.array_equal(outs[l - 1]["V_log"], V)


def test_single_chunk_has_zero_deviation():
    """A one-chunk prompt sits at the same positions in compile and link:
    d == 0 for every token, S is empty, nothing is selected."""
    w = wl.tiny(n_layers=2, lens=(96,))
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    K1, _ = OL.splice(req, compiled, 1)
    st, out = OL.wca_layer1(req, w.shape, E, W(1), K1, k_cap=24)
    assert np.all(out["d"] == 0.0) and st.S_k == [] and st.ranking == []
    assert np.all(out["alpha"] == 0.0)


def test_first_chunk_zero_deviation_in_multichunk_prompt():
    w = wl.tiny(n_layers=2, lens=(40, 24, 36), dtype="bf16")
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    K1, _ = OL.splice(req, compiled, 1)
    _, out = OL.wca_layer1(req, w.shape, E, W(1), K1, k_cap=20)
    assert np.all(out["d"][:40] == 0.0)
    assert np.all(out["d"][40:] > 0.0)
    assert all(i >= 40 for i in out["S_k"])


# ------------------------------------------------------------ layer-1 closed forms

def _pre_rope_keys(w, E, W, tokens):
    s = w.shape
    Wl = {k: torch.tensor(v) for k, v in W(1).items()}
    a = F.rms_norm(torch.tensor(E[tokens]), (s.d_model,), weight=Wl["norm1"], eps=s.rms_eps)
    y = a @ Wl["w_qkv"].T
    return y[:, s.q_dim: s.q_dim + s.kv_dim].view(len(tokens), s.n_kv_heads, s.head_dim).numpy()


def test_layer1_deviation_alpha_cksim_closed_forms():
    """Under RoPE, layer-1 keys of a token differ between compile and link only
    by a rotation of each pair by the chunk offset D (CacheSlide PMKD discussion):
      d = sum_h sum_j 2 |z_hj|^2 (1 - cos(D theta_j)),  alpha = d / sum |z|^2,
      cos_h = sum_j |z_hj|^2 cos(D theta_j) / sum_j |z_hj|^2."""
    w = tiny64(n_layers=1, lens=(40, 24, 36))
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    K1, V1 = OL.splice(req, compiled, 1)
    _, out = OL.wca_layer1(req, w.shape, E, W(1), K1, k_cap=20)
    z = _pre_rope_keys(w, E, W, req.tokens)
    hd = w.shape.head_dim
    half = hd // 2
    zz = z[..., :half] ** 2 + z[..., half:] ** 2                   # [N, H, half]
    theta = 10000.0 ** (-2.0 * np.arange(half) / hd)
    D = np.concatenate([np.full(len(c), s) for s, c in zip(req.chunk_starts, req.chunks)])
    cosD = np.cos(D[:, None] * theta[None, :])[:, None, :]
    d_ref = (2 * zz * (1 - cosD)).sum(axis=(1, 2))
    assert np.allclose(out["d"], d_ref, rtol=1e-9, atol=1e-12)
    assert np.allclose(out["alpha"], d_ref / zz.sum(axis=(1, 2)), rtol=1e-9, atol=1e-12)
    assert np.all((out["alpha"] >= 0) & (out["alpha"] <= 4))
    cos_ref = ((zz * cosD).sum(-1) / zz.sum(-1)).mean(-1)
    assert np.allclose(OS.cksim(out["k"], K1), cos_ref, rtol=1e-9, atol=1e-12)
    # values carry no rotation: layer-1 V is recomputed bit for bit
    assert np.array_equal(out["v"], V1)


# ------------------------------------------------------------ blend / alpha / cksim

def test_blend_and_alpha_closed_forms(rng):
    rec = rng.standard_normal((9, 2, 8))
    reu = rng.standard_normal((9, 2, 8))
    d = OS.deviation(rec, reu)
    n = OS.row_sq(reu)
    a = OS.alpha_of(d, n)
    assert np.allclose(a * n, d, rtol=1e-14)
    out = OS.blend(a, rec, reu)
    assert np.allclose(out - reu, a[:, None, None] * (rec - reu), atol=1e-13)
    assert np.array_equal(OS.blend(np.zeros(9), rec, reu), reu)
    assert np.array_equal(OS.blend(np.ones(9), rec, reu), rec)
    assert np.all(OS.deviation(reu, reu) == 0) and np.all(OS.alpha_of(OS.deviation(reu, reu), n) == 0)
    z = np.zeros((2, 2, 8))
    assert list(OS.alpha_of(OS.deviation(rec[:2], z), OS.row_sq(z))) == [1.0, 1.0]
    assert list(OS.alpha_of(np.zeros(2), np.zeros(2))) == [0.0, 0.0]


def test_cksim_special_values(rng):
    x = rng.standard_normal((4, 3, 16))
    assert np.allclose(OS.cksim(x, x), 1.0)
    assert np.allclose(OS.cksim(x, -x), -1.0)
    y = x.copy()
    y[:, 0] *= -1           # one head reversed out of three
    assert np.allclose(OS.cksim(x, y), 1.0 / 3.0)
    e1 = np.zeros((1, 1, 4)); e1[0, 0, 0] = 1
    e2 = np.zeros((1, 1, 4)); e2[0, 0, 1] = 2
    assert OS.cksim(e1, e2)[0] == 0.0
    assert OS.cksim(np.zeros((1, 1, 4)), np.zeros((1, 1, 4)))[0] == 1.0
    assert OS.cksim(e1, np.zeros((1, 1, 4)))[0] == 0.0


# ------------------------------------------------------------ top-k (brute force)

def _brute_topk(d, k):
    """The unique k-subset of S = {d > 0} that no outside element beats
    (larger d, or equal d and lower index)."""
    S = [i for i in range(len(d)) if d[i] > 0]
    k = min(k, len(S))
    found = []
    for sub in itertools.combinations(S, k):
        inside = set(sub)
        ok = all(not (d[o] > d[i] or (d[o] == d[i] and o < i)) for o in S if o not in inside for i in sub)
        if ok:
            found.append(sorted(sub))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("case", range(60))
def test_top_k_brute_force(case):
    g = np.random.default_rng(case)
    n = int(g.integers(1, 11))
    d = g.choice([0.0, 0.5, 1.0, 2.0, 3.5], size=n) if case % 2 else np.abs(g.standard_normal(n)) * (g.random(n) > 0.3)
    k = int(g.integers(0, n + 2))
    rk, sk, cur = OS.top_k(d, k)
    assert sk == _brute_topk(d, k)
    assert cur == len(sk) == min(k, int((d > 0).sum()))
    assert sorted(rk) == [i for i in range(n) if d[i] > 0]
    for a, b in zip(rk, rk[1:]):
        assert d[a] > d[b] or (d[a] == d[b] and a < b)


# ------------------------------------------------------------ refresh (hand-worked golden cases)

def test_refresh_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "refresh_cases.json")))["cases"]
    for c in cases:
        S_next, cur, retired = OS.refresh(c["S_k"], np.array(c["c"]), c["tau"], c["ranking"], c["cursor"], c["rule"])
        assert S_next == c["S_next"], c["name"]
        assert cur == c["cursor_next"], c["name"]
        assert sorted(retired) == c["retired"], c["name"]


# ------------------------------------------------------------ page tables (hand-worked example)

def test_page_tables_tiny_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "pages_tiny.json")))
    w = wl.tiny()
    req = w.requests[0]
    alloc = OP.PageAllocator(4096)
    plan = OP.compile_plan(w.compile_chunks, 2, alloc)
    assert {str(k): v for k, v in plan.items()} == g["compile_pages"]
    link = [alloc.alloc(OP.n_pages_for(OP.capacity("cacheslide", 512, 0.26, 0, l))) for l in (1, 2)]
    assert link == g["link_pages"]
    for s in g["reuse_slot_samples"]:
        assert OP.reuse_slots(req, plan, s["layer"])[s["token"]] == s["slot"]
    for s in g["new_slot_samples"]:
        assert OP.slot_of(link[s["layer"] - 1], s["rank"]) == s["slot"]


def test_allocator_lowest_first_and_capacity():
    a = OP.PageAllocator(10)
    assert a.alloc(3) == [0, 1, 2]
    assert a.alloc(2) == [3, 4]
    a.release([1, 3])
    assert a.alloc(3) == [1, 3, 5]
    with pytest.raises(OP.CapacityError):
        a.alloc(5)
    sm = OP.slot_map(np.arange(100, 110), np.array([2, 5, 7]), [40])
    assert list(sm) == [100, 101, 640, 103, 104, 641, 106, 642, 108, 109]


# ------------------------------------------------------------ the alpha order (a reading, checked for consistency)

def test_wca_alpha_lag_and_refresh_consistency():
    """alpha used at layer l is the alpha computed at the token's previous
    recompute (layer 1 for a fresh token); refills come from the ranking."""
    w = wl.tiny(n_layers=9)
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    k_cap = int(np.floor(0.26 * req.n_tokens))
    # a threshold inside the spread of CKSim so that both branches run
    st, outs = OL.wca_link(req, w.shape, E, W, compiled, k_cap, tau=0.2)
    last_alpha = dict(enumerate(outs[0]["alpha"]))
    seen_retire = False
    for l in range(2, 10):
        o = outs[l - 1]
        for t, i in enumerate(o["S"]):
            assert o["alpha_used"][t] == last_alpha[int(i)]
            last_alpha[int(i)] = o["alpha_new"][t]
        if "retired" in o:
            seen_retire |= len(o["retired"]) > 0
            new = set(o["S_next"]) - set(int(i) for i in o["S"])
            assert new <= set(st.ranking)
            assert not (set(o["retired"]) & set(o["S_next"]))
    assert seen_retire


# ------------------------------------------------------------ refresh timing and the stale carry (hand-worked)

def test_refresh_schedule_golden():
    g = json.load(open(os.path.join(GOLDEN, "refresh_timing.json")))
    for c in g["schedules"]:
        assert OL.refresh_layers(c["n_layers"], c["period"]) == c["gates_after"], c


@pytest.mark.parametrize("case", [0, 1])
def test_all_retire_schedule_and_stale_carry(case):
    """Every token retires at every gate: the oracle's set of each layer is the
    golden's ranking slice, the gate runs exactly after the golden's layers,
    and a token that joins enters with layer 1's output, checked against the
    library decoder's first layer over the spliced prompt."""
    gold = json.load(open(os.path.join(GOLDEN, "refresh_timing.json")))
    g = gold["all_retire"]
    c = g["cases"][case]
    L = c["n_layers"]
    w = tiny64(n_layers=L, lens=(40, 60, 60, 60))
    E, W = oracle_inputs(w)
    req = w.requests[0]
    compiled = OL.compile_chunks(w.compile_chunks, w.shape, E, W)
    k = int(np.floor(0.26 * req.n_tokens))
    st, outs = OL.wca_link(req, w.shape, E, W, compiled, k, tau=g["tau"], period=c["period"], rule=g["rule"])
    ranking = outs[0]["ranking"]
    assert len(ranking) >= 3 * k
    gated = [l for l in range(2, L + 1) if "cksim" in outs[l - 1]]
    sched = [x for x in gold["schedules"] if x["n_layers"] == L and x["period"] == c["period"]]
    assert gated == sched[0]["gates_after"]
    for l in range(2, L + 1):
        lo, hi = c["rank_slices"][str(l)]
        assert list(outs[l - 1]["S"]) == sorted(ranking[lo * k: hi * k]), l
    _, _, h1 = torch_prefill(req.tokens, w.shape, E, W, 1)
    for l in c["fresh_layers"]:
        S = outs[l - 1]["S"]
        assert np.allclose(outs[l - 1]["h_in"], h1[S], rtol=1e-10, atol=1e-10), l
    # a layer that is not the first after a gate starts from the previous layer's output rows
    for l in range(3, L + 1):
        if l not in c["fresh_layers"]:
            prev = outs[l - 2]
            assert np.array_equal(outs[l - 1]["S"], prev["S"])
            assert np.array_equal(outs[l - 1]["h_in"], prev["h_rows"])


# ------------------------------------------------------------ SLIDE dirty-page counters (hand-worked)

def test_dirty_counts_and_spill_order_golden():
    g = json.load(open(os.path.join(GOLDEN, "dirty_pages.json")))
    rq = g["request"]
    ch = lambda uid, n: wl.Chunk(uid=uid, kind="fixed", tokens=np.zeros(n, dtype=np.int32))
    req = wl.Request([ch(i, n) for i, n in enumerate(rq["chunks"])])
    L, N = rq["n_layers"], req.n_tokens
    alloc = OP.PageAllocator(rq["n_pages"])
    plan = OP.compile_plan(req.chunks, L, alloc)
    assert {str(k): v for k, v in plan.items()} == g["compile_pages"]
    new = {l: alloc.alloc(len(g["new_pages"][str(l)])) for l in range(1, L + 1)}
    assert {str(l): p for l, p in new.items()} == g["new_pages"]
    routes = []
    for l in range(1, L + 1):
        S = np.arange(N) if g["selected"][str(l)] == "all" else np.asarray(g["selected"][str(l)])
        sm = OP.slot_map(OP.reuse_slots(req, plan, l), S, new[l])
        if l > 1:
            assert list(sm[S]) == g["new_slots_worked"][str(l)]
        routes.append((sm, S))
    # overwrite-first decode placement: the reused slots of each layer's recomputed tokens, in token order
    n_dec = g["decode_tokens"]
    dec = []
    for l, (sm, S) in enumerate(routes, start=1):
        dec += list(OP.reuse_slots(req, plan, l)[np.sort(S)][:n_dec])
    assert dec == g["decode_slots_worked"]["slots"]
    want_link = np.zeros(rq["n_pages"], dtype=np.int64)
    for p, c in g["counts_after_link"].items():
        want_link[int(p)] = c
    assert np.array_equal(OP.dirty_counts(rq["n_pages"], routes), want_link)
    want = np.zeros(rq["n_pages"], dtype=np.int64)
    for p, c in g["counts_after_decode"].items():
        want[int(p)] = c
    counts = OP.dirty_counts(rq["n_pages"], routes, dec)
    assert np.array_equal(counts, want)
    assert OP.spill_order(counts, range(rq["n_pages"])) == g["spill_order_after_decode"]

