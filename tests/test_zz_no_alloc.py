"""The allocation-free top-k entry point (kvb_deviation_topk_noalloc) against
kvb_deviation_topk with a caller workspace: two calls in a row, the second on
a smaller batch, every output bitwise equal (the same kernels; only where the
sort keys live differs); the first call's outputs also against the oracle.
Sizes past the fixed scratch are refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import select as OS
from selective_kv_cache_amd import _lib as K
from helpers import np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPE = wl.ModelShape(n_layers=1, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536, dtype="bf16")


def i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)


def case(g, req_lens):
    s = SHAPE
    B, n_tok = len(req_lens), sum(req_lens)
    cu = np.concatenate([[0], np.cumsum(req_lens)]).astype(np.int64)
    n_pages = (n_tok + 15) // 16 + 2
    kp = torch.tensor(g.standard_normal((n_pages, s.n_kv_heads, 16, s.head_dim)), dtype=torch.float32)
    kp = kp.to(torch.bfloat16)
    reuse_slot = g.permutation(n_pages * 16)[:n_tok]
    idx = torch.as_tensor(reuse_slot)
    k_rec = kp[idx // 16, :, idx % 16, :].float()
    k_rec += 0.3 * torch.tensor(g.standard_normal(k_rec.shape), dtype=torch.float32)
    for b in range(B):   # each request's first 40 tokens reproduce the cache: d == 0
        n0 = min(40, req_lens[b])
        k_rec[cu[b]:cu[b] + n0] = kp[idx[cu[b]:cu[b] + n0] // 16, :, idx[cu[b]:cu[b] + n0] % 16, :].float()
    k_cap = [int(np.floor(0.26 * n)) for n in req_lens]
    return dict(B=B, n_tok=n_tok, cu=cu, n_pages=n_pages, kp=kp.to(DEV), reuse_slot=reuse_slot,
                k_rec=k_rec.to(torch.bfloat16).to(DEV), k_cap=k_cap)


def outputs(c):
    n, B = c["n_tok"], c["B"]
    return dict(d=torch.full((n,), -1.0, device=DEV), alpha=torch.full((n,), -1.0, device=DEV),
                ranking=torch.full((n,), -7, dtype=torch.int32, device=DEV),
                s_count=torch.full((B,), -7, dtype=torch.int32, device=DEV),
                sel=torch.full((n,), -7, dtype=torch.int32, device=DEV),
                cu_rows=torch.full((B + 1,), -7, dtype=torch.int32, device=DEV),
                cursor=torch.full((B,), -7, dtype=torch.int32, device=DEV))


def run(ctx, c, noalloc):
    desc = K.model_desc(SHAPE)
    o = outputs(c)
    args = (ctx, K.stream_handle(), desc, c["B"], c["n_tok"], i32(c["cu"]), c["k_rec"], c["kp"], c["n_pages"],
            i32(c["reuse_slot"]), i32(c["k_cap"]), o["d"], o["alpha"], o["ranking"], o["s_count"], o["sel"],
            o["cu_rows"], o["cursor"])
    if noalloc:
        K.kvb_deviation_topk_noalloc(*args)
    else:
        wsb = K.kvb_workspace_size(ctx, desc, 1, c["n_tok"], c["B"])
        ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device=DEV)
        K.kvb_deviation_topk(*args, ws, wsb)
    torch.cuda.synchronize()
    return o


@pytest.fixture(scope="module")
def ctx():
    c = K.kvb_create(0)
    yield c
    K.kvb_destroy(c)


def test_noalloc_matches_workspace_call_twice(ctx):
    g = np.random.default_rng(5)
    big = case(g, [9000, 300, 2049, 64, 17000])
    small = case(g, [700, 33])
    for c in (big, small):     # the second call reuses the scratch left by the first
        ref = run(ctx, c, noalloc=False)
        got = run(ctx, c, noalloc=True)
        for k in ref:
            assert torch.equal(got[k], ref[k]), k
    # the first call's results against the oracle: d and the exact top-k of that d
    c, o = big, run(ctx, big, noalloc=True)
    idx = torch.as_tensor(c["reuse_slot"], device=DEV)
    reuse = np64(c["kp"][idx // 16, :, idx % 16, :])
    gd = np64(o["d"])
    assert np.allclose(gd, OS.deviation(np64(c["k_rec"]), reuse), rtol=2e-5, atol=0)
    sel, cr = o["sel"].cpu().numpy(), o["cu_rows"].cpu().numpy()
    for b in range(c["B"]):
        seg = slice(c["cu"][b], c["cu"][b + 1])
        _, S_k, _ = OS.top_k(gd[seg], c["k_cap"][b])
        assert list(sel[cr[b]:cr[b + 1]] - c["cu"][b]) == S_k


def test_noalloc_refuses_batches_past_its_scratch(ctx):
    desc = K.model_desc(SHAPE)
    one = torch.zeros(8, dtype=torch.int32, device=DEV)
    f = torch.zeros(8, device=DEV)
    with pytest.raises(K.KvbError) as e:
        K.kvb_deviation_topk_noalloc(ctx, K.stream_handle(), desc, 1, K.KVB_NOALLOC_MAX_TOKENS + 1, one, one, one, 1,
                                     one, one, f, f, one, one, one, one, one)
    assert e.value.status == K.KVB_ERR_WORKSPACE
    with pytest.raises(K.KvbError) as e:
        K.kvb_deviation_topk_noalloc(ctx, K.stream_handle(), desc, K.KVB_NOALLOC_MAX_REQUESTS + 1, 8, one, one, one,
                                     1, one, one, f, f, one, one, one, one, one)
    assert e.value.status == K.KVB_ERR_WORKSPACE
