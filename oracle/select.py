"""Selection, fusion and refresh of Weighted Correction Attention (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

All from the CacheSlide page, "Method details", the cross-layer KV similarity /
Weighted Correction Attention paragraphs and Algorithm 2:
  * per-token squared deviation  d_i = ||K_i^rec - K_i^reuse||^2 ;
  * S = {i : d_i > 0}; S_k = the k tokens of S with the largest d ;
  * fusion  K_i <- alpha_i K_i^rec + (1 - alpha_i) K_i^reuse (same for V) with
    alpha_i = ||K_i^rec - K_i^reuse||^2 / ||K_i^reuse||^2 ;
  * every four layers, c_i = CKSim(K_i^rec, K_i^reuse) (mean over heads of the
    cosine, "Background", PMKD paragraph); a token with c_i < tau leaves S_k
    and S, and the token of S \\ S_k with the largest d joins S_k.

Readings (the pages leave these open):
  * d and alpha are per token over the whole key row (all KV heads x head_dim);
  * ties in d are broken by the lower token index; S_k is kept ascending;
  * alpha is not clamped; if ||K^reuse||^2 == 0, alpha = 0 when d == 0, else 1;
  * the refresh looks at a snapshot of S_k; refills take the next unused
    entries of the layer-1 ranking (d only exists at layer 1), so retired
    tokens never return; if the ranking runs out S_k shrinks;
  * a KV head whose two vectors are both zero has cosine 1, one zero vector 0.

CacheBlend-style selection (EPIC page, section 3.2, the CacheBlend baseline:
layer 1 recomputes every token, the attention maps computed with the old
(cached) and the new (recomputed) KV are compared, and the tokens whose maps
differ most, 15 %, are recomputed in the later layers):
  * a token's deviation is the L1 distance between its two attention rows,
    averaged over the query heads (reading: the page names no distance; L1 is
    the plain distance between two probability rows and lies in [0, 2]);
  * both rows use the layer-1 queries recomputed at the spliced positions
    (the cache holds no queries), the causal key range of the token, and the
    model's 1/sqrt(hd) scale; the selection then follows the same ranking,
    S = {dev > 0} and top-k rule as above.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def row_sq(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return (x.reshape(x.shape[0], -1) ** 2).sum(axis=1)


def deviation(k_rec: np.ndarray, k_reuse: np.ndarray) -> np.ndarray:
    """d_i = ||K_i^rec - K_i^reuse||^2 over the full key row, float64 [T]."""
    return row_sq(np.asarray(k_rec, dtype=np.float64) - np.asarray(k_reuse, dtype=np.float64))


def alpha_of(d: np.ndarray, reuse_sq: np.ndarray) -> np.ndarray:
    """alpha_i = d_i / ||K_i^reuse||^2 with the zero-denominator reading."""
    d = np.asarray(d, dtype=np.float64)
    n = np.asarray(reuse_sq, dtype=np.float64)
    out = np.where(d == 0.0, 0.0, 1.0)
    nz = n > 0
    out[nz] = d[nz] / n[nz]
    return out


def ranking_of(d: np.ndarray) -> List[int]:
    """Tokens of S = {d > 0} ordered by d descending, ties by lower index."""
    d = np.asarray(d)
    S = [i for i in range(d.shape[0]) if d[i] > 0]
    return sorted(S, key=lambda i: (-float(d[i]), i))


def top_k(d: np.ndarray, k_cap: int) -> Tuple[List[int], List[int], int]:
    """(ranking, S_k ascending, cursor) with k = min(k_cap, |S|)."""
    rk = ranking_of(d)
    k = min(int(k_cap), len(rk))
    return rk, sorted(rk[:k]), k


def blend(alpha: np.ndarray, x_rec: np.ndarray, x_reuse: np.ndarray) -> np.ndarray:
    """alpha * x_rec + (1 - alpha) * x_reuse, alpha broadcast per row (float64)."""
    a = np.asarray(alpha, dtype=np.float64).reshape(-1, *([1] * (np.ndim(x_rec) - 1)))
    return a * np.asarray(x_rec, dtype=np.float64) + (1.0 - a) * np.asarray(x_reuse, dtype=np.float64)


def cksim(k_rec: np.ndarray, k_reuse: np.ndarray) -> np.ndarray:
    """Mean over KV heads of cos(K^rec_h, K^reuse_h); rows [T, H, hd] -> [T]."""
    a = np.asarray(k_rec, dtype=np.float64)
    b = np.asarray(k_reuse, dtype=np.float64)
    dot = (a * b).sum(axis=-1)
    na = np.sqrt((a * a).sum(axis=-1))
    nb = np.sqrt((b * b).sum(axis=-1))
    both0 = (na == 0) & (nb == 0)
    one0 = (na == 0) ^ (nb == 0)
    den = np.where((na > 0) & (nb > 0), na * nb, 1.0)
    cos = np.where(both0, 1.0, np.where(one0, 0.0, dot / den))
    return cos.mean(axis=-1)


def refresh(S_k: List[int], c: np.ndarray, tau: float, ranking: List[int], cursor: int,
            rule: str = "literal") -> Tuple[List[int], int, List[int]]:
    """Similarity-gated retire/refill on a snapshot of S_k.

    c[j] is CKSim of S_k[j].  rule "literal": retire when c < tau (the pages'
    stated test); rule "dissim": retire when c > 1 - tau.  Returns
    (new S_k ascending, new cursor, retired tokens).
    """
    c = np.asarray(c, dtype=np.float64)
    if rule == "literal":
        retire = [S_k[j] for j in range(len(S_k)) if c[j] < tau]
    elif rule == "dissim":
        retire = [S_k[j] for j in range(len(S_k)) if c[j] > 1.0 - tau]
    else:
        raise ValueError(rule)
    gone = set(retire)
    keep = [i for i in S_k if i not in gone]
    n_new = min(len(retire), len(ranking) - cursor)
    refill = ranking[cursor: cursor + n_new]
    return sorted(keep + refill), cursor + n_new, retire


def attention_map_deviation(q: np.ndarray, k_new: np.ndarray, k_old: np.ndarray, lo: np.ndarray,
                            shape, rows=None) -> np.ndarray:
    """Per-token attention-map deviation of the CacheBlend-style selection.

    q [N, Hq, hd] layer-1 queries at the spliced positions; k_new, k_old
    [N, Hkv, hd] the recomputed and the cached (spliced) layer-1 keys; lo [N]
    the first key a token may see.  For token i and query head h (KV head
    h // (Hq / Hkv)) the two attention rows are softmax over keys j in
    lo_i..i of q_i . k_j / sqrt(hd), once with k_new and once with k_old;
    the result is the mean over h of the L1 distance of the two rows, float64 [N]
    (or, with `rows`, for those tokens only, in that order).
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    k_old = np.asarray(k_old, dtype=np.float64)
    N, Hq, hd = q.shape
    G = Hq // k_new.shape[1]
    scale = 1.0 / np.sqrt(hd)
    rows = range(N) if rows is None else [int(i) for i in rows]
    dev = np.zeros(len(rows))
    for t, i in enumerate(rows):
        j0 = int(lo[i])
        total = 0.0
        for h in range(Hq):
            rows = []
            for K in (k_new, k_old):
                s = K[j0:i + 1, h // G] @ q[i, h] * scale
                e = np.exp(s - s.max())
                rows.append(e / e.sum())
            total += np.abs(rows[0] - rows[1]).sum()
        dev[t] = total / Hq
    return dev
