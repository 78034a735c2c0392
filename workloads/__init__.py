"""Seeded synthetic workloads for the link step of position-independent KV reuse.

This module is shared by the CPU oracle's tests and by the GPU path. It holds
configuration records and seeded random draws (chunk lengths, token ids,
embedding table, weights) and nothing else: no step of the method's arithmetic
lives here, so that the oracle and the kernels stay independent.

Workload shapes follow the pages' agent / RAG prompts: a prompt is a list of
chunks that alternate between "fixed" (reused, e.g. a system prefix or a
retrieved document) and "dynamic" (per-request) segments.  Each chunk is
compiled alone from position 0; the link step splices them (CacheSlide page,
"Background" on agent prompt structure; EPIC page, section 3.1 compile/link).

Random streams (numpy SeedSequence keys ``[seed, stream, ...]``):
  1 token ids per chunk uid, 2 chunk lengths, 3 embedding table,
  4 weights per (layer, matrix), 5 per-request draws of the batched workload.
Large tensors (embedding, weights) are drawn with torch's Philox generator on
the requested device, seeded from the SeedSequence key, so that the GPU tests
can generate multi-GB weight sets in place; a CPU test that needs the same
values copies them from wherever they were generated.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

VOCAB = 32000

# matrix ids inside the weight stream
W_QKV, W_O, W_GATE_UP, W_DOWN = 0, 1, 2, 3


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    dtype: str = "bf16"          # "fp32" or "bf16": storage type of weights, KV, hidden state
    rope_base: float = 10000.0
    rms_eps: float = 1e-5
    page_size: int = 16
    vocab: int = VOCAB
    weight_std: float = 0.02

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    def params_per_layer(self) -> int:
        d = self.d_model
        return self.qkv_rows * d + d * self.q_dim + 3 * d * self.ffn


@dataclass
class Chunk:
    uid: int                     # identity of the compiled instance (shared fixed chunks share it)
    kind: str                    # "fixed", "dynamic", or "query" (mutable tokens that are never compiled)
    tokens: np.ndarray           # int32 [len]

    def __len__(self) -> int:
        return int(self.tokens.shape[0])

    @property
    def cached(self) -> bool:
        """True when the chunk has compile-step KV to reuse."""
        return self.kind != "query"


@dataclass
class Request:
    chunks: List[Chunk]

    @property
    def n_tokens(self) -> int:
        return sum(len(c) for c in self.chunks)

    @property
    def chunk_starts(self) -> List[int]:
        out, s = [], 0
        for c in self.chunks:
            out.append(s)
            s += len(c)
        return out

    @property
    def tokens(self) -> np.ndarray:
        return np.concatenate([c.tokens for c in self.chunks]).astype(np.int32)


@dataclass
class Workload:
    name: str
    shape: ModelShape
    mode: str                    # "cacheslide", "legolink" or "cacheblend"
    requests: List[Request]
    ratio: float = 0.26          # top-k ratio (CacheSlide; the CacheBlend-style selection uses cb_ratio)
    cb_ratio: float = 0.15       # CacheBlend-style selection ratio
    tau: float = 0.12            # CKSim threshold
    period: int = 4              # refresh every `period` layers
    lego_k: int = 32             # LegoLink first-k per chunk
    seed: int = 0
    gen_device: str = "cpu"      # where embedding / weights are drawn
    notes: str = ""

    @property
    def compile_chunks(self) -> List[Chunk]:
        """Unique chunk instances in compile order (first appearance)."""
        seen, out = set(), []
        for req in self.requests:
            for c in req.chunks:
                if c.cached and c.uid not in seen:
                    seen.add(c.uid)
                    out.append(c)
        return out

    @property
    def n_tokens_total(self) -> int:
        return sum(r.n_tokens for r in self.requests)


# --------------------------------------------------------------------------
# seeded draws
# --------------------------------------------------------------------------

def rng(seed: int, stream: int, *ids: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, *ids]))


def torch_seed(seed: int, stream: int, *ids: int) -> int:
    st = np.random.SeedSequence([seed, stream, *ids]).generate_state(2, np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


def chunk_tokens(seed: int, uid: int, n: int) -> np.ndarray:
    return rng(seed, 1, uid).integers(0, VOCAB, size=n, dtype=np.int64).astype(np.int32)


def draw_lengths_fixed_sum(g: np.random.Generator, n: int, lo: int, hi: int, total: int) -> List[int]:
    """n-1 iid U{lo..hi}, last = total - sum; redraw until last lies in [lo, hi]."""
    while True:
        head = g.integers(lo, hi + 1, size=n - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return [int(x) for x in head] + [last]


def alternating_kinds(n: int) -> List[str]:
    return ["fixed" if i % 2 == 0 else "dynamic" for i in range(n)]


def _single_request(seed: int, lens: List[int], query_len: int = 0) -> Request:
    """Alternating fixed / dynamic chunks, then (query_len > 0) an uncached query suffix."""
    kinds = alternating_kinds(len(lens))
    chunks = [Chunk(uid=i, kind=kinds[i], tokens=chunk_tokens(seed, i, n)) for i, n in enumerate(lens)]
    if query_len > 0:
        u = len(lens)
        chunks.append(Chunk(uid=u, kind="query", tokens=chunk_tokens(seed, u, query_len)))
    return Request(chunks)


def gen_normal(shape, std: float, key: int, device: str = "cpu", dtype: str = "fp32"):
    """N(0, std^2) tensor from torch's generator on `device`, rounded to `dtype` storage."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(key)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    return x


def embedding_table(w: Workload, device: Optional[str] = None):
    s = w.shape
    return gen_normal((s.vocab, s.d_model), 1.0, torch_seed(w.seed, 3), device or w.gen_device, s.dtype)


def layer_weights(w: Workload, layer: int, device: Optional[str] = None) -> dict:
    """Weights of 1-based `layer`: w_qkv [(Hq+2Hkv)hd, d], w_o [d, Hq hd],
    w_gate_up [2F, d] (gate rows then up rows), w_down [d, F], norm1/norm2 [d] = 1."""
    import torch
    s, dev = w.shape, device or w.gen_device
    d, F = s.d_model, s.ffn
    out = {
        "w_qkv": gen_normal((s.qkv_rows, d), s.weight_std, torch_seed(w.seed, 4, layer, W_QKV), dev, s.dtype),
        "w_o": gen_normal((d, s.q_dim), s.weight_std, torch_seed(w.seed, 4, layer, W_O), dev, s.dtype),
        "w_gate_up": gen_normal((2 * F, d), s.weight_std, torch_seed(w.seed, 4, layer, W_GATE_UP), dev, s.dtype),
        "w_down": gen_normal((d, F), s.weight_std, torch_seed(w.seed, 4, layer, W_DOWN), dev, s.dtype),
    }
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    out["norm1"] = torch.ones(d, device=dev, dtype=tdt)
    out["norm2"] = torch.ones(d, device=dev, dtype=tdt)
    return out


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------

TINY = ModelShape(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688, dtype="fp32")
MISTRAL = ModelShape(n_layers=32, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336, dtype="bf16")
LLAMA70 = ModelShape(n_layers=80, d_model=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, ffn=28672, dtype="bf16")


def tiny(seed: int = 0, n_layers: int = 2, lens=(128, 96, 160, 128), mode: str = "cacheslide",
         dtype: str = "fp32", query_len: int = 0, **kw) -> Workload:
    """Tiny decoder: 4 chunks [fixed 128, dynamic 96, fixed 160, dynamic 128], fp32."""
    shape = ModelShape(**{**TINY.__dict__, "n_layers": n_layers, "dtype": dtype})
    return Workload(f"tiny-{n_layers}L", shape, mode, [_single_request(seed, list(lens), query_len)], seed=seed,
                    **kw)


def small_bf16(seed: int = 0, n_layers: int = 8, lens=(192, 320, 256, 288), mode: str = "cacheslide",
               head_dim: int = 128, query_len: int = 0, **kw) -> Workload:
    """A small bf16 stack with the large configs' head geometry (GQA 4, hd 128),
    sized so that the oracle finishes in seconds while kernels still span several tiles."""
    shape = ModelShape(n_layers=n_layers, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=head_dim,
                       ffn=1536, dtype="bf16")
    return Workload(f"small-bf16-{n_layers}L", shape, mode, [_single_request(seed, list(lens), query_len)],
                    seed=seed, **kw)


def mistral_cacheslide(seed: int = 0, n_layers: int = 32) -> Workload:
    """Mistral-7B-shaped stack, one 8192-token request of 8 alternating chunks U[512,1536]."""
    lens = draw_lengths_fixed_sum(rng(seed, 2, 0), 8, 512, 1536, 8192)
    shape = ModelShape(**{**MISTRAL.__dict__, "n_layers": n_layers})
    return Workload("mistral7b-cacheslide-8k", shape, "cacheslide", [_single_request(seed, lens)],
                    seed=seed, gen_device="cuda")


def mistral_legolink(seed: int = 0, n_layers: int = 32, query_len: int = 0) -> Workload:
    """Mistral-7B-shaped stack, 16384 tokens as 32 chunks of 512, LegoLink k=32
    (query_len > 0: then an uncached query of that many tokens)."""
    shape = ModelShape(**{**MISTRAL.__dict__, "n_layers": n_layers})
    name = "mistral7b-legolink-16k" + (f"-q{query_len}" if query_len else "")
    return Workload(name, shape, "legolink", [_single_request(seed, [512] * 32, query_len)],
                    seed=seed, gen_device="cuda")


def mistral_batch8(seed: int = 0, n_layers: int = 32, n_requests: int = 8) -> Workload:
    """Batch of 8 requests, N_r ~ U{4096..16384}, 6..12 alternating chunks; six shared
    fixed chunks (U{128..512}) reused across requests, dynamic chunks redrawn per request."""
    g = rng(seed, 2, 100)
    fixed_lens = [int(x) for x in g.integers(128, 513, size=6)]
    fixed = [Chunk(uid=i, kind="fixed", tokens=chunk_tokens(seed, i, n)) for i, n in enumerate(fixed_lens)]
    reqs = []
    uid = 1000
    for r in range(n_requests):
        gr = rng(seed, 5, r)
        while True:
            n_tok = int(gr.integers(4096, 16385))
            n_ch = int(gr.integers(6, 13))
            n_fix, n_dyn = (n_ch + 1) // 2, n_ch // 2
            dyn_total = n_tok - sum(fixed_lens[:n_fix])
            if dyn_total >= max(1024, 64 * n_dyn):
                break
        extra = dyn_total - 64 * n_dyn
        cuts = sorted(int(x) for x in gr.integers(0, extra + 1, size=n_dyn - 1))
        dyn_lens = [b - a + 64 for a, b in zip([0] + cuts, cuts + [extra])]
        chunks = []
        for i in range(n_ch):
            if i % 2 == 0:
                chunks.append(fixed[i // 2])
            else:
                n = dyn_lens[i // 2]
                chunks.append(Chunk(uid=uid, kind="dynamic", tokens=chunk_tokens(seed, uid, n)))
                uid += 1
        reqs.append(Request(chunks))
    shape = ModelShape(**{**MISTRAL.__dict__, "n_layers": n_layers})
    return Workload("mistral7b-cacheslide-batch8", shape, "cacheslide", reqs, seed=seed, gen_device="cuda")


def llama70_cacheslide(seed: int = 0, n_layers: int = 80) -> Workload:
    """Llama-3-70B-shaped stack, one 32768-token request of 16 alternating chunks U[1024,3072]."""
    lens = draw_lengths_fixed_sum(rng(seed, 2, 0), 16, 1024, 3072, 32768)
    shape = ModelShape(**{**LLAMA70.__dict__, "n_layers": n_layers})
    return Workload("llama70b-cacheslide-32k", shape, "cacheslide", [_single_request(seed, lens)],
                    seed=seed, gen_device="cuda")


NAMED = {
    "tiny": tiny,
    "mistral7b-cacheslide-8k": mistral_cacheslide,
    "mistral7b-legolink-16k": mistral_legolink,
    "mistral7b-cacheslide-batch8": mistral_batch8,
    "llama70b-cacheslide-32k": llama70_cacheslide,
}
