"""Decoder-layer arithmetic of the oracle, in float64 numpy.

TEST INFRASTRUCTURE ONLY: the oracle is a plain, slow CPU statement of what the
link step computes.  Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the product path never does.

Model (the pages fix none of it beyond the configuration shapes; this is the
plain reading used throughout): RMSNorm -> Q,K,V projections without bias ->
rotate-half RoPE -> causal grouped-query attention with scale 1/sqrt(hd) ->
output projection + residual -> RMSNorm -> SwiGLU MLP + residual.  The
LegoLink derivation on the EPIC page (section 4, "LegoLink" steps 1-5) gives
the same per-layer dataflow for the recomputed rows: Q,K,V = E W, expanded K/V
over all N tokens, A = softmax(Q K_exp^T masked causally), O = A V_exp W_O.

Storage precision: every tensor handed from one step to the next (q, k, v
after RoPE, blended K/V, attention output, residual stream, MLP intermediate)
is rounded to the storage type (float32, or bfloat16 with round-to-nearest-
even); arithmetic inside a step is float64.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- storage

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as float64.

    Goes through float32 first (round-to-nearest-even), then drops the low 16
    bits of the float32 pattern with round-half-to-even on the dropped part.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value as held in memory by a path running in `dtype`.

    "bf16" and "fp32" are the two storage types of the method's paths; "fp64"
    keeps float64 (no rounding) and serves the closed-form checks.
    """
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- pieces

def rmsnorm(h: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: h / sqrt(mean(h^2) + eps) * g."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """Angle p * base^(-2j/hd) for pair j = 0..hd/2-1, float64, shape [T, hd/2]."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * j / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE of x [T, H, hd] at integer positions pos [T].

    Pair (j, j + hd/2) is rotated by angle p * theta_j:
      y_j        = x_j cos - x_{j+hd/2} sin
      y_{j+hd/2} = x_{j+hd/2} cos + x_j sin
    """
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    ang = rope_angles(pos, hd, base)[:, None, :]            # [T, 1, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def project_rows(a: np.ndarray, w: np.ndarray, blocks=None) -> np.ndarray:
    """a [T, d] @ w^T with w [n_out, d].

    `blocks` (list of (start, stop)) splits the rows into separately issued
    products.  Compile and link issue layer-1 projections with identical
    per-chunk row blocks so that a chunk seen at the same positions in both
    gets bitwise-identical keys (its layer-1 deviation is then exactly 0).
    """
    a = np.asarray(a, dtype=np.float64)
    wt = np.asarray(w, dtype=np.float64).T
    if blocks is None:
        return a @ wt
    out = np.empty((a.shape[0], wt.shape[1]), dtype=np.float64)
    for s, e in blocks:
        out[s:e] = a[s:e] @ wt
    return out


def qkv(h: np.ndarray, pos: np.ndarray, W: dict, shape, blocks=None):
    """RMSNorm + Q/K/V projection + RoPE for rows h [T, d] at positions pos [T].

    Returns (q [T,Hq,hd], k [T,Hkv,hd], v [T,Hkv,hd]) rounded to storage.
    """
    s = shape
    a = rmsnorm(h, W["norm1"], s.rms_eps)
    y = project_rows(a, W["w_qkv"], blocks)
    T = h.shape[0]
    q = y[:, : s.q_dim].reshape(T, s.n_q_heads, s.head_dim)
    k = y[:, s.q_dim: s.q_dim + s.kv_dim].reshape(T, s.n_kv_heads, s.head_dim)
    v = y[:, s.q_dim + s.kv_dim:].reshape(T, s.n_kv_heads, s.head_dim)
    q = rope(q, pos, s.rope_base)
    k = rope(k, pos, s.rope_base)
    return store(q, s.dtype), store(k, s.dtype), store(v, s.dtype)


def attention_rows(q: np.ndarray, qpos: np.ndarray, K: np.ndarray, V: np.ndarray, lo: np.ndarray,
                   shape) -> np.ndarray:
    """Causal grouped-query attention for query rows only.

    q [T, Hq, hd] are the queries of tokens at positions qpos [T] (indices into
    K/V); K, V [N, Hkv, hd] are the layer's full logical keys/values.  Query t
    attends keys j with lo[t] <= j <= qpos[t].  Head h reads KV head
    h // (Hq / Hkv).  Plain softmax in float64.  Returns [T, Hq*hd] (storage).
    """
    s = shape
    G = s.n_q_heads // s.n_kv_heads
    scale = 1.0 / np.sqrt(s.head_dim)
    T = q.shape[0]
    out = np.zeros((T, s.n_q_heads, s.head_dim), dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    for t in range(T):
        p0, p1 = int(lo[t]), int(qpos[t])
        for h in range(s.n_q_heads):
            kh = h // G
            sc = K[p0:p1 + 1, kh, :] @ q[t, h, :] * scale
            sc = sc - sc.max()
            e = np.exp(sc)
            out[t, h, :] = (e / e.sum()) @ V[p0:p1 + 1, kh, :]
    return store(out.reshape(T, -1), s.dtype)


def attention_rows_fast(q, qpos, K, V, lo, shape):
    """Same result as attention_rows, computed per head with a masked matrix product.

    Used for whole layers where the per-row loop would be slow; the tests pin
    it to attention_rows and to torch's reference attention.
    """
    s = shape
    G = s.n_q_heads // s.n_kv_heads
    scale = 1.0 / np.sqrt(s.head_dim)
    T = q.shape[0]
    N = K.shape[0]
    keys = np.arange(N)
    mask = (keys[None, :] <= np.asarray(qpos)[:, None]) & (keys[None, :] >= np.asarray(lo)[:, None])
    out = np.zeros((T, s.n_q_heads, s.head_dim), dtype=np.float64)
    for h in range(s.n_q_heads):
        kh = h // G
        sc = (np.asarray(q[:, h, :], dtype=np.float64) @ np.asarray(K[:, kh, :], dtype=np.float64).T) * scale
        sc = np.where(mask, sc, -np.inf)
        sc = sc - sc.max(axis=1, keepdims=True)
        e = np.exp(sc)
        out[:, h, :] = (e / e.sum(axis=1, keepdims=True)) @ np.asarray(V[:, kh, :], dtype=np.float64)
    return store(out.reshape(T, -1), s.dtype)


def post_attention(h: np.ndarray, o: np.ndarray, W: dict, shape) -> np.ndarray:
    """h + o W_o^T, then h' + SwiGLU(RMSNorm(h')): returns the new residual rows."""
    s = shape
    h1 = store(np.asarray(h, dtype=np.float64) + project_rows(o, W["w_o"]), s.dtype)
    b = rmsnorm(h1, W["norm2"], s.rms_eps)
    gu = project_rows(b, W["w_gate_up"])
    F = s.ffn
    u = store(silu(gu[:, :F]) * gu[:, F:], s.dtype)
    return store(h1 + project_rows(u, W["w_down"]), s.dtype)
