"""Compile and link steps of position-independent KV reuse (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Compile (EPIC page, section 3.1 and "System Overview"): each immutable chunk is
prefilled on its own with positions starting from zero and its per-layer K/V
are kept.  Link: the cached K/V of a request's chunks are spliced (token i of
the request at global position i) and a subset of tokens is recomputed.

Three ways of choosing that subset are implemented:
  * CacheSlide Weighted Correction Attention (CacheSlide page, "Method
    details" and Algorithm 2): layer 1 recomputes every token, then the k
    tokens with the largest key deviation are recomputed in layers 2..L and
    fused with the cached K/V; every four layers a cosine check retires and
    refills tokens;
  * EPIC LegoLink (EPIC page, section 4 "LegoLink"): a static set, the first k
    tokens of every chunk except the first plus the uncached query tokens,
    recomputed in every layer, whose K/V replace the cached ones;
  * the CacheBlend baseline as the EPIC page describes it (section 3.2): layer 1
    recomputes every token, the 15 % whose attention maps deviate most from the
    cached ones are recomputed in layers 2..L and replace the cached K/V.
"Fully recompute" and "Naive" (EPIC page, section 3.2) are the static-set
cases S = everything and S = nothing.

Readings taken where the pages are silent (each is listed with its reason in
the design notes): keys are compared after RoPE and cached keys keep their
chunk-local rotation; layer 1's K/V are the recomputed ones (fusion starts at
layer 2); alpha used at layer l is the token's alpha from the last layer it was
recomputed in, then alpha is updated from layer l (Algorithm 2's order); the
refresh runs after layer l when l % 4 == 0 and l < L and changes the set from
layer l+1; a refilled token carries its last computed hidden state (for a
token not recomputed since layer 1, layer 1's output); selected rows attend
causally over the full spliced KV of the layer, including their own fused K/V.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np

from . import model as M
from . import select as Sel


def as_f64(x) -> np.ndarray:
    """torch tensor (any device / dtype) or array -> float64 numpy."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- prefill

def full_prefill(tokens: np.ndarray, shape, E: np.ndarray, W: Callable[[int], dict],
                 n_layers: Optional[int] = None, skip_last_mlp: bool = False, lo: int = 0):
    """Standard causal forward of `tokens` at positions 0..N-1.

    Returns (K list, V list, final hidden [N, d]); K[l-1] is layer l's
    post-RoPE keys.  With skip_last_mlp the last layer's attention and MLP,
    which no cached K/V depends on, are not evaluated (final hidden is None).
    """
    L = n_layers or shape.n_layers
    N = len(tokens)
    pos = np.arange(N)
    h = M.store(E[np.asarray(tokens)], shape.dtype)
    Ks, Vs = [], []
    for l in range(1, L + 1):
        Wl = W(l)
        q, k, v = M.qkv(h, pos, Wl, shape)
        Ks.append(k)
        Vs.append(v)
        if skip_last_mlp and l == L:
            return Ks, Vs, None
        o = M.attention_rows_fast(q, pos, k, v, np.full(N, lo), shape)
        h = M.post_attention(h, o, Wl, shape)
    return Ks, Vs, h


def compile_chunks(chunks, shape, E, W) -> Dict[int, tuple]:
    """uid -> (K list, V list) for every cached chunk instance, each prefilled alone.
    A query chunk (the request's mutable tokens) has no compile step."""
    out = {}
    for c in chunks:
        if not c.cached:
            continue
        K, V, _ = full_prefill(c.tokens, shape, E, W, skip_last_mlp=True)
        out[c.uid] = (K, V)
    return out


def splice(request, compiled: Dict[int, tuple], layer: int, shape=None):
    """Request's reuse K, V at 1-based `layer`: the chunks' cached rows concatenated.

    Rows of an uncached query chunk are NaN: such tokens are recomputed in every
    layer, so their cached rows must never be read (a NaN would show if they were)."""
    def rows(c, i):
        if c.cached:
            return compiled[c.uid][i][layer - 1]
        if shape is not None:
            tail = (shape.n_kv_heads, shape.head_dim)
        else:
            tail = next(iter(compiled.values()))[i][layer - 1].shape[1:]
        return np.full((len(c),) + tuple(tail), np.nan)

    K = np.concatenate([rows(c, 0) for c in request.chunks])
    V = np.concatenate([rows(c, 1) for c in request.chunks])
    return K, V


def chunk_blocks(request):
    s = request.chunk_starts
    return [(a, a + len(c)) for a, c in zip(s, request.chunks)]


# ---------------------------------------------------------------- CacheSlide

def refresh_layers(n_layers: int, period: int) -> List[int]:
    """Layers after which the similarity gate runs (1-based).

    The CacheSlide page (Algorithm 2) checks CKSim every fourth layer.  The
    gate after layer l changes the set used from layer l+1 on, so a gate after
    the last layer would change nothing: it runs after l = period, 2*period, ...
    with l < n_layers.
    """
    return list(range(period, n_layers, period))


@dataclass
class WCAState:
    """Per-request state of Weighted Correction Attention between layers.

    Rows of `h` outside the current set keep the last value computed for them:
    a token that joins the set at a refresh enters with the output of the last
    layer that recomputed it (layer 1 for a token never selected before)."""
    h: np.ndarray                 # [N, d] residual stream
    alpha: np.ndarray             # [N] correction weight of each token's latest recompute
    d: np.ndarray                 # [N] layer-1 deviation
    ranking: List[int]            # tokens with d > 0, largest d first (ties: lower index)
    cursor: int                   # ranking entries used so far
    S_k: List[int]                # the set recomputed by the next layer, ascending
    layer: int = 1                # last layer done


def wca_layer1(request, shape, E, W1: dict, reuse_K1: np.ndarray, k_cap: int):
    """Layer 1: full recompute of every token at its spliced position, deviation,
    alpha and top-k selection.  Returns (state, outputs)."""
    tokens = request.tokens
    N = len(tokens)
    pos = np.arange(N)
    h = M.store(E[tokens], shape.dtype)
    q, k, v = M.qkv(h, pos, W1, shape, blocks=chunk_blocks(request))
    o = M.attention_rows_fast(q, pos, k, v, np.zeros(N, dtype=np.int64), shape)
    h2 = M.post_attention(h, o, W1, shape)
    d = Sel.deviation(k, reuse_K1)
    alpha = Sel.alpha_of(d, Sel.row_sq(reuse_K1))
    ranking, S_k, cursor = Sel.top_k(d, k_cap)
    out = dict(q=q, k=k, v=v, o=o, h=h2.copy(), d=d, alpha=alpha, ranking=ranking, S_k=S_k, cursor=cursor)
    return WCAState(h=h2, alpha=alpha.copy(), d=d, ranking=ranking, cursor=cursor, S_k=S_k), out


def corrected_cache(S: np.ndarray, k_rec, v_rec, reuse_K, reuse_V, weight: np.ndarray, dtype: str):
    """The layer's logical K/V after the weighted correction of the rows S.

    Rows S hold weight * recomputed + (1 - weight) * cached (the fusion of the
    CacheSlide page, one value of the weight per token for K and V alike),
    rounded once to storage; every other row is the cached one.
    Returns (K, V, fused K rows, fused V rows)."""
    Kb = M.store(Sel.blend(weight, k_rec, reuse_K[S]), dtype)
    Vb = M.store(Sel.blend(weight, v_rec, reuse_V[S]), dtype)
    K = np.array(reuse_K, dtype=np.float64, copy=True)
    V = np.array(reuse_V, dtype=np.float64, copy=True)
    K[S] = Kb
    V[S] = Vb
    return K, V, Kb, Vb


def wca_layer(state: WCAState, layer: int, shape, W: dict, reuse_K: np.ndarray, reuse_V: np.ndarray,
              gate: bool, tau: float = 0.12, alpha_mode: str = "lag", rule: str = "literal",
              attn_rows: Optional[np.ndarray] = None):
    """One layer l >= 2 for the tokens of S_k.  Mutates `state`; returns outputs.

    The rows of S_k are recomputed from their current hidden state; their
    deviation from the cached keys gives this layer's alpha.  The cache of the
    layer is corrected with the alpha the token carried into the layer (its
    latest one; `alpha_mode` "current" uses this layer's, "one" plain
    replacement), the selected rows attend over it and their residual stream
    advances.  With `gate` the similarity check then updates S_k for the next
    layer.  attn_rows (indices into S_k) limits attention, MLP and the hidden
    update to a sample of rows (full-size checks); the cache, alpha and the
    gate always cover all of S_k.
    """
    S = np.asarray(state.S_k, dtype=np.int64)
    h_in = state.h[S].copy()
    q, k, v = M.qkv(h_in, S, W, shape)
    kr = reuse_K[S]
    d_l = Sel.deviation(k, kr)
    a_new = Sel.alpha_of(d_l, Sel.row_sq(kr))
    a_use = {"lag": lambda: state.alpha[S].copy(), "current": lambda: a_new,
             "one": lambda: np.ones_like(a_new)}[alpha_mode]()
    K_log, V_log, Kb, Vb = corrected_cache(S, k, v, reuse_K, reuse_V, a_use, shape.dtype)
    state.alpha[S] = a_new
    rows = np.arange(S.size) if attn_rows is None else np.asarray(attn_rows, dtype=np.int64)
    o = M.attention_rows_fast(q[rows], S[rows], K_log, V_log, np.zeros(rows.size, dtype=np.int64), shape)
    h_rows = M.post_attention(h_in[rows], o, W, shape)
    state.h[S[rows]] = h_rows
    out = dict(S=S, h_in=h_in, q=q, k_rec=k, v_rec=v, K_blend=Kb, V_blend=Vb, d=d_l, alpha_used=a_use,
               alpha_new=a_new, o=o, h_rows=h_rows, rows=rows, K_log=K_log, V_log=V_log)
    if gate:
        c = Sel.cksim(k, kr)
        S_next, cur, retired = Sel.refresh(state.S_k, c, tau, state.ranking, state.cursor, rule)
        state.S_k, state.cursor = S_next, cur
        out.update(cksim=c, retired=retired)
    out.update(S_next=list(state.S_k), cursor=state.cursor)
    state.layer = layer
    return out


def wca_link(request, shape, E, W, compiled, k_cap: int, tau: float, period: int = 4,
             alpha_mode: str = "lag", rule: str = "literal", keep: bool = True):
    """Free-running CacheSlide link step of one request.  Returns (state, per-layer outputs)."""
    L = shape.n_layers
    gates = set(refresh_layers(L, period))
    K1, _ = splice(request, compiled, 1)
    state, out1 = wca_layer1(request, shape, E, W(1), K1, k_cap)
    outs = [out1]
    for l in range(2, L + 1):
        Kl, Vl = splice(request, compiled, l)
        o = wca_layer(state, l, shape, W(l), Kl, Vl, l in gates, tau, alpha_mode, rule)
        outs.append(o if keep else {k: o[k] for k in ("S", "h_rows", "S_next")})
    return state, outs


# ---------------------------------------------------------------- CacheBlend-style selection

def cacheblend_layer1(request, shape, E, W1: dict, reuse_K1: np.ndarray, k_cap: int):
    """Layer 1 of the CacheBlend-style link (EPIC page, section 3.2): every token
    recomputed at its spliced position (the KV written is the recomputed one),
    then the attention-map deviation of every token against the cached keys
    and the top-k of S = {dev > 0}.  Returns (state, outputs); alpha is 1 for
    every token: the later layers' recomputed KV replace the cached KV."""
    tokens = request.tokens
    N = len(tokens)
    pos = np.arange(N)
    h = M.store(E[tokens], shape.dtype)
    q, k, v = M.qkv(h, pos, W1, shape, blocks=chunk_blocks(request))
    o = M.attention_rows_fast(q, pos, k, v, np.zeros(N, dtype=np.int64), shape)
    h2 = M.post_attention(h, o, W1, shape)
    dev = Sel.attention_map_deviation(q, k, reuse_K1, np.zeros(N, dtype=np.int64), shape)
    ranking, S_k, cursor = Sel.top_k(dev, k_cap)
    out = dict(q=q, k=k, v=v, o=o, h=h2.copy(), d=dev, ranking=ranking, S_k=S_k, cursor=cursor)
    return WCAState(h=h2, alpha=np.ones(N), d=dev, ranking=ranking, cursor=cursor, S_k=S_k), out


def cacheblend_link(request, shape, E, W, compiled, k_cap: int, keep: bool = True):
    """CacheBlend-style link of one request: layer 1 as above, then layers 2..L
    recompute the fixed set S_k (no refresh) and its KV replaces the cache."""
    L = shape.n_layers
    K1, _ = splice(request, compiled, 1)
    state, out1 = cacheblend_layer1(request, shape, E, W(1), K1, k_cap)
    outs = [out1]
    for l in range(2, L + 1):
        Kl, Vl = splice(request, compiled, l)
        o = wca_layer(state, l, shape, W(l), Kl, Vl, gate=False, alpha_mode="one")
        outs.append(o if keep else {k: o[k] for k in ("S", "h_rows", "S_next")})
    return state, outs


# ---------------------------------------------------------------- static sets

def legolink_rows(request, k: int) -> np.ndarray:
    """LegoLink's static set (EPIC page, section 4): the first min(k, len) tokens
    of every cached chunk except the first, plus every token of the request's
    uncached query chunks (the user's mutable input, which has no cache)."""
    rows = []
    for c, ((s, e), ch) in enumerate(zip(chunk_blocks(request), request.chunks)):
        if not ch.cached:
            rows.extend(range(s, e))
        elif c > 0:
            rows.extend(range(s, s + min(k, e - s)))
    return np.asarray(rows, dtype=np.int64)


def static_link(request, S: np.ndarray, shape, E, W, compiled, keep: bool = True):
    """Recompute the fixed set S (ascending) in every layer; its K/V replace the cached ones.

    Returns (hidden rows of S after the last layer [|S|, d], per-layer outputs)."""
    tokens = request.tokens
    S = np.asarray(S, dtype=np.int64)
    hS = M.store(E[tokens[S]], shape.dtype)
    outs = []
    for l in range(1, shape.n_layers + 1):
        Wl = W(l)
        Kr, Vr = splice(request, compiled, l, shape)
        K_log = np.array(Kr, dtype=np.float64, copy=True)
        V_log = np.array(Vr, dtype=np.float64, copy=True)
        if S.size:
            q, k, v = M.qkv(hS, S, Wl, shape)
            K_log[S] = k
            V_log[S] = v
            o = M.attention_rows_fast(q, S, K_log, V_log, np.zeros(S.size, dtype=np.int64), shape)
            hS = M.post_attention(hS, o, Wl, shape)
        else:
            q = k = v = o = None
        outs.append(dict(S=S, q=q, k=k, v=v, o=o, h_rows=hS, K_log=K_log, V_log=V_log) if keep
                    else dict(S=S, h_rows=hS))
    return hS, outs
