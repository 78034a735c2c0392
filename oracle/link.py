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

@dataclass
class WCAState:
    """Per-request state of Weighted Correction Attention between layers."""
    h: np.ndarray                 # [N, d] residual stream (stale rows keep their last value)
    alpha: np.ndarray             # [N]
    d: np.ndarray                 # [N] layer-1 deviation
    ranking: List[int]
    cursor: int
    S_k: List[int]                # ascending
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


def wca_layer(state: WCAState, layer: int, shape, W: dict, reuse_K: np.ndarray, reuse_V: np.ndarray,
              tau: float, period: int, n_layers: int, alpha_mode: str = "lag", rule: str = "literal",
              attn_rows: Optional[np.ndarray] = None):
    """One layer l >= 2 for the tokens of S_k.  Mutates `state`; returns outputs.

    attn_rows (indices into S_k) limits attention, MLP and the hidden update to
    a sample of rows (used at full size); fusion, alpha and the refresh always
    cover all of S_k.
    """
    S = np.asarray(state.S_k, dtype=np.int64)
    q, k, v = M.qkv(state.h[S], S, W, shape)
    kr, vr = reuse_K[S], reuse_V[S]
    d_l = Sel.deviation(k, kr)
    a_new = Sel.alpha_of(d_l, Sel.row_sq(kr))
    if alpha_mode == "lag":
        a_use = state.alpha[S].copy()
    elif alpha_mode == "current":
        a_use = a_new
    elif alpha_mode == "one":          # alpha forced to 1: plain recompute (pin only)
        a_use = np.ones_like(a_new)
    else:
        raise ValueError(alpha_mode)
    Kb = M.store(Sel.blend(a_use, k, kr), shape.dtype)
    Vb = M.store(Sel.blend(a_use, v, vr), shape.dtype)
    K_log = np.array(reuse_K, dtype=np.float64, copy=True)
    V_log = np.array(reuse_V, dtype=np.float64, copy=True)
    K_log[S] = Kb
    V_log[S] = Vb
    rows = np.arange(S.size) if attn_rows is None else np.asarray(attn_rows, dtype=np.int64)
    o = M.attention_rows_fast(q[rows], S[rows], K_log, V_log, np.zeros(rows.size, dtype=np.int64), shape)
    h_rows = M.post_attention(state.h[S[rows]], o, W, shape)
    state.h[S[rows]] = h_rows
    state.alpha[S] = a_new
    out = dict(S=S, q=q, k_rec=k, v_rec=v, K_blend=Kb, V_blend=Vb, d=d_l, alpha_used=a_use,
               alpha_new=a_new, o=o, h_rows=h_rows, rows=rows, K_log=K_log, V_log=V_log)
    if layer % period == 0 and layer < n_layers:
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
    K1, _ = splice(request, compiled, 1)
    state, out1 = wca_layer1(request, shape, E, W(1), K1, k_cap)
    outs = [out1]
    for l in range(2, L + 1):
        Kl, Vl = splice(request, compiled, l)
        o = wca_layer(state, l, shape, W(l), Kl, Vl, tau, period, L, alpha_mode, rule)
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
        o = wca_layer(state, l, shape, W(l), Kl, Vl, tau=0.0, period=L + 1, n_layers=L, alpha_mode="one")
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
