"""Per-entry-point parity of the HIP kernels against the CPU oracle (GPU).

Every call goes through the C ABI (ctypes).  Inputs are seeded and sized to
span several tiles with ragged tails; device-side row counts smaller than the
launch bound check that rows past the count are left untouched.
"""
import numpy as np
import pytest
import torch

from selective_kv_cache_amd import _lib as K
from oracle import model as OM
from oracle import pages as OP
from oracle import select as OS
import workloads as wl
from helpers import TOL, max_rel_err, np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SHAPES = {
    "bf16": wl.ModelShape(n_layers=1, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536, dtype="bf16"),
    "bf16_hd64": wl.ModelShape(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=1, head_dim=64, ffn=512, dtype="bf16"),
    # wide enough that a one-row product runs whole 4-chunk batches per lane
    # (d = 2048) and a ragged tail (ffn = 2816)
    "bf16_wide": wl.ModelShape(n_layers=1, d_model=2048, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=2816,
                               dtype="bf16"),
    "fp32": wl.ModelShape(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688, dtype="fp32"),
    # a row of 320 16-byte chunks: in the one-row products' normalising
    # staging some threads take two chunks and the others one
    "bf16_ragged": wl.ModelShape(n_layers=1, d_model=2560, n_q_heads=20, n_kv_heads=4, head_dim=128, ffn=6912,
                                 dtype="bf16"),
}


@pytest.fixture(scope="module")
def ctx():
    c = K.kvb_create(0)
    yield c
    K.kvb_destroy(c)


def tdt(shape):
    return torch.bfloat16 if shape.dtype == "bf16" else torch.float32


def rand(shape_, g, std=1.0, s=None, dtype=None):
    x = torch.tensor(g.standard_normal(shape_) * std, dtype=torch.float32)
    return x.to(dtype) if dtype is not None else x


def i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=DEV)


def sh():
    return K.stream_handle()


def workspace(ctx, desc, T_max, n_tok=1, B=1):
    wsb = K.kvb_workspace_size(ctx, desc, T_max, n_tok, B)
    return torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV), wsb


def weights(shape, g):
    d, F = shape.d_model, shape.ffn
    dt = tdt(shape)
    W = {
        "w_qkv": rand((shape.qkv_rows, d), g, 0.02, dtype=dt),
        "w_o": rand((d, shape.q_dim), g, 0.02, dtype=dt),
        "w_gate_up": rand((2 * F, d), g, 0.02, dtype=dt),
        "w_down": rand((d, F), g, 0.02, dtype=dt),
        "norm1": (1.0 + 0.1 * rand((d,), g)).to(dt),
        "norm2": (1.0 + 0.1 * rand((d,), g)).to(dt),
    }
    return {k: v.to(DEV) for k, v in W.items()}


# ------------------------------------------------------------------ Q/K/V projection + RoPE

@pytest.mark.parametrize("name", ["bf16", "bf16_hd64", "bf16_wide", "fp32"])
@pytest.mark.parametrize("flags,T_max,n_valid", [(K.KVB_QKV_BATCH_INVARIANT, 200, 173), (K.KVB_QKV_SPLIT_K, 200, 173),
                                                 (K.KVB_QKV_SPLIT_K, 7, 5), (K.KVB_QKV_SPLIT_K, 1, 1)])
def test_qkv_proj_rope(ctx, name, flags, T_max, n_valid):
    s = SHAPES[name]
    g = np.random.default_rng(11)
    desc = K.model_desc(s)
    n_tok = 300
    dt = tdt(s)
    hidden = rand((n_tok, s.d_model), g, dtype=dt).to(DEV)
    W = weights(s, g)
    rows = np.sort(g.choice(n_tok, T_max, replace=False))
    pos = g.integers(0, 32768, n_tok)
    q = torch.full((T_max, s.n_q_heads, s.head_dim), 7.0, dtype=dt, device=DEV)
    k = torch.full((T_max, s.n_kv_heads, s.head_dim), 7.0, dtype=dt, device=DEV)
    v = torch.full((T_max, s.n_kv_heads, s.head_dim), 7.0, dtype=dt, device=DEV)
    ws, wsb = workspace(ctx, desc, T_max)
    K.kvb_timing_enable(ctx, "splitk")
    K.kvb_qkv_proj(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows), hidden, W["norm1"], W["w_qkv"], i32(pos),
                   q, k, v, ws, wsb, flags)
    split = "splitk_reduce" in K.kvb_timing_read(ctx)
    K.kvb_timing_enable(ctx, None)
    torch.cuda.synchronize()
    # the batch-invariant projection never splits K; nor does a single row
    # that may (it takes the one-row weight-streaming product)
    if flags == K.KVB_QKV_BATCH_INVARIANT or s.dtype == "fp32" or T_max == 1:
        assert not split
    Wn = {kk: np64(vv) for kk, vv in W.items()}
    rq, rk, rv = OM.qkv(np64(hidden)[rows[:n_valid]], pos[rows[:n_valid]], Wn, s)
    assert max_rel_err(q[:n_valid], rq) < TOL[s.dtype]
    assert max_rel_err(k[:n_valid], rk) < TOL[s.dtype]
    assert max_rel_err(v[:n_valid], rv) < TOL[s.dtype]
    assert torch.all(q[n_valid:] == 7.0) and torch.all(k[n_valid:] == 7.0) and torch.all(v[n_valid:] == 7.0)


@pytest.mark.parametrize("name", ["bf16", "fp32"])
def test_qkv_rows_are_batch_invariant(ctx, name):
    """A row's projection is bitwise the same whatever batch and tile slot it sits in."""
    s = SHAPES[name]
    g = np.random.default_rng(5)
    desc = K.model_desc(s)
    dt = tdt(s)
    n_tok = 400
    hidden = rand((n_tok, s.d_model), g, dtype=dt).to(DEV)
    W = weights(s, g)
    pos = i32(g.integers(0, 5000, n_tok))
    outs = []
    for rows in (np.arange(0, 150), np.concatenate([np.arange(250, 400), np.arange(0, 150)])):
        T = len(rows)
        q = torch.empty((T, s.n_q_heads, s.head_dim), dtype=dt, device=DEV)
        k = torch.empty((T, s.n_kv_heads, s.head_dim), dtype=dt, device=DEV)
        v = torch.empty((T, s.n_kv_heads, s.head_dim), dtype=dt, device=DEV)
        ws, wsb = workspace(ctx, desc, T)
        K.kvb_qkv_proj(ctx, sh(), desc, T, None, i32(rows), hidden, W["norm1"], W["w_qkv"], pos, q, k, v, ws, wsb)
        outs.append((q, k, v))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a[:150], b[150:300])


def test_rope_standalone(ctx):
    s = SHAPES["bf16"]
    g = np.random.default_rng(3)
    desc = K.model_desc(s)
    T = 70
    q0 = rand((T, s.n_q_heads, s.head_dim), g, dtype=torch.bfloat16)
    k0 = rand((T, s.n_kv_heads, s.head_dim), g, dtype=torch.bfloat16)
    pos = g.integers(0, 32768, T)
    q, k = q0.to(DEV), k0.to(DEV)
    K.kvb_rope(ctx, sh(), desc, T, None, None, i32(pos), q, k)
    torch.cuda.synchronize()
    assert max_rel_err(q, OM.rope(np64(q0), pos, 1e4)) < 8e-3
    assert max_rel_err(k, OM.rope(np64(k0), pos, 1e4)) < 8e-3


# ------------------------------------------------------------------ fusion + scatter

def _pool(s, n_pages, g):
    dt = tdt(s)
    kp = rand((n_pages, s.n_kv_heads, 16, s.head_dim), g, dtype=dt).to(DEV)
    vp = rand((n_pages, s.n_kv_heads, 16, s.head_dim), g, dtype=dt).to(DEV)
    return kp, vp


def _rows_at(pool, slots, s):
    p = np64(pool)
    slots = np.asarray(slots)
    return p[slots // 16, :, slots % 16, :]


@pytest.mark.parametrize("name", ["bf16", "fp32", "bf16_hd64"])
@pytest.mark.parametrize("mode", [K.KVB_ALPHA_LAG, K.KVB_ALPHA_CURRENT, K.KVB_ALPHA_ONE])
def test_blend_scatter(ctx, name, mode):
    s = SHAPES[name]
    g = np.random.default_rng(21 + mode)
    desc = K.model_desc(s)
    dt = tdt(s)
    n_pages, n_tok, T_max, n_valid = 48, 500, 150, 131
    kp, vp = _pool(s, n_pages, g)
    kp0, vp0 = kp.clone(), vp.clone()
    perm = g.permutation(n_pages * 16)
    src_slot = perm[:n_tok]                          # token -> cached slot
    rows = np.sort(g.choice(n_tok, T_max, replace=False))
    dst = perm[n_tok:n_tok + T_max]                  # fresh slots, disjoint from the cached ones
    k_rec = rand((T_max, s.n_kv_heads, s.head_dim), g, dtype=dt)
    v_rec = rand((T_max, s.n_kv_heads, s.head_dim), g, dtype=dt)
    # special rows: identical to the cache (d = 0), and a zero cached key (zero denominator)
    reuse_k = _rows_at(kp0, src_slot[rows], s)
    k_rec[3] = torch.tensor(reuse_k[3], dtype=torch.float32).to(dt)
    kp[src_slot[rows[5]] // 16, :, src_slot[rows[5]] % 16, :] = 0
    reuse_k = _rows_at(kp, src_slot[rows], s)
    reuse_v = _rows_at(vp, src_slot[rows], s)
    alpha0 = g.uniform(-0.5, 2.0, n_tok).astype(np.float32)
    alpha0[rows[7]] = 0.0
    alpha0[rows[8]] = 1.0
    alpha = torch.tensor(alpha0, device=DEV)
    d_out = torch.full((T_max,), -1.0, device=DEV)
    ck = torch.full((T_max,), -9.0, device=DEV)
    K.kvb_blend_scatter(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows), k_rec.to(DEV), v_rec.to(DEV), kp, vp,
                        n_pages, i32(src_slot), i32(dst), mode, alpha, d_out, ck)
    torch.cuda.synchronize()
    n = n_valid
    kr, vr = np64(k_rec)[:n], np64(v_rec)[:n]
    d_ref = OS.deviation(kr, reuse_k[:n])
    a_new = OS.alpha_of(d_ref, OS.row_sq(reuse_k[:n]))
    a_use = {K.KVB_ALPHA_LAG: alpha0[rows[:n]].astype(np.float64), K.KVB_ALPHA_CURRENT: a_new,
             K.KVB_ALPHA_ONE: np.ones(n)}[mode]
    kb = OM.store(OS.blend(a_use, kr, reuse_k[:n]), s.dtype)
    vb = OM.store(OS.blend(a_use, vr, reuse_v[:n]), s.dtype)
    assert max_rel_err(_rows_at(kp, dst[:n], s), kb) < TOL[s.dtype]
    assert max_rel_err(_rows_at(vp, dst[:n], s), vb) < TOL[s.dtype]
    got_d = np64(d_out)
    assert np.allclose(got_d[:n], d_ref, rtol=2e-5, atol=1e-6) and got_d[3] == 0.0
    assert np.all(got_d[n:] == -1.0)
    a_got = np64(alpha)
    if mode == K.KVB_ALPHA_ONE:
        assert np.array_equal(a_got, alpha0.astype(np.float64))
    else:
        assert np.allclose(a_got[rows[:n]], a_new, rtol=2e-5, atol=1e-7)
        assert a_got[rows[3]] == 0.0 and a_got[rows[5]] == 1.0
    assert np.allclose(np64(ck)[:n], OS.cksim(kr, reuse_k[:n]), atol=2e-5)
    # alpha = 0 keeps the cached row exactly, alpha = 1 the recomputed one (stored)
    if mode == K.KVB_ALPHA_LAG:
        assert np.array_equal(_rows_at(kp, dst[7:8], s), reuse_k[7:8])
        assert np.array_equal(_rows_at(kp, dst[8:9], s), OM.store(kr[8:9], s.dtype))
    # nothing else in the pools moved
    touched = np.zeros(n_pages * 16, bool)
    touched[dst[:n]] = True
    touched[src_slot[rows[5]]] = True
    untouched = np.flatnonzero(~touched)
    assert np.array_equal(_rows_at(kp, untouched, s), _rows_at(kp0, untouched, s))


@pytest.mark.parametrize("name", ["bf16", "bf16_hd64", "bf16_wide", "bf16_ragged", "fp32"])
@pytest.mark.parametrize("mode,cached", [(K.KVB_ALPHA_LAG, True), (K.KVB_ALPHA_ONE, True), (K.KVB_ALPHA_ONE, False),
                                         (K.KVB_ALPHA_CURRENT, True)], ids=["lag", "one", "one-nocache", "current"])
@pytest.mark.parametrize("flags,T_max,n_valid", [(K.KVB_QKV_BATCH_INVARIANT, 200, 173), (K.KVB_QKV_SPLIT_K, 200, 173),
                                                 (K.KVB_QKV_SPLIT_K, 1, 1)], ids=["inv", "splitk", "one-row"])
def test_qkv_fused(ctx, name, mode, cached, flags, T_max, n_valid):
    """Projection, then RoPE + fusion + scatter in one pass (for one bf16 row
    with nothing cached, as in decode, inside the product's epilogue): bitwise
    the result of kvb_qkv_proj (with positions) followed by kvb_blend_scatter
    on the same inputs; Q/K/V against the oracle, and the fused rows, d, alpha
    and CKSim against the oracle applied to the call's own recomputed K/V."""
    s = SHAPES[name]
    g = np.random.default_rng(31 + mode + 7 * T_max)
    desc = K.model_desc(s)
    dt = tdt(s)
    n_tok, n_pages = 300, 64
    hidden = rand((n_tok, s.d_model), g, dtype=dt).to(DEV)
    W = weights(s, g)
    rows = np.sort(g.choice(n_tok, T_max, replace=False))
    pos = g.integers(0, 32768, n_tok)
    kp, vp = _pool(s, n_pages, g)
    perm = g.permutation(n_pages * 16)
    src_slot = perm[:n_tok]
    dst = perm[n_tok:n_tok + T_max].copy()
    if T_max > 1:
        dst[4] = -1                                   # a row with no new slot: nothing scattered
        kp[src_slot[rows[6]] // 16, :, src_slot[rows[6]] % 16, :] = 0   # a zero cached key
    kp0, vp0 = kp.clone(), vp.clone()
    alpha0 = g.uniform(-0.5, 2.0, n_tok).astype(np.float32)
    alpha0[rows[0]] = 1.0
    ws, wsb = workspace(ctx, desc, T_max, n_tok)

    def run(fused):
        o = dict(q=torch.full((T_max, s.n_q_heads, s.head_dim), 7.0, dtype=dt, device=DEV),
                 k=torch.full((T_max, s.n_kv_heads, s.head_dim), 7.0, dtype=dt, device=DEV),
                 v=torch.full((T_max, s.n_kv_heads, s.head_dim), 7.0, dtype=dt, device=DEV),
                 kp=kp0.clone(), vp=vp0.clone(), alpha=torch.tensor(alpha0, device=DEV),
                 d=torch.full((T_max,), -1.0, device=DEV), ck=torch.full((T_max,), -9.0, device=DEV))
        blend = (o["kp"], o["vp"], n_pages, i32(src_slot) if cached else None, i32(dst), mode,
                 o["alpha"] if cached else None, o["d"] if cached else None, o["ck"] if cached else None)
        if fused:
            K.kvb_timing_enable(ctx, "")
            K.kvb_qkv_fused(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows), hidden, W["norm1"], W["w_qkv"],
                            i32(pos), o["q"], o["k"], o["v"], *blend, ws, wsb, flags)
            o["launched"] = K.kvb_timing_read(ctx)
            K.kvb_timing_enable(ctx, None)
        else:
            K.kvb_qkv_proj(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows), hidden, W["norm1"], W["w_qkv"],
                           i32(pos), o["q"], o["k"], o["v"], ws, wsb, flags)
            K.kvb_blend_scatter(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows), o["k"], o["v"], *blend)
        torch.cuda.synchronize()
        return o

    ref, got = run(False), run(True)
    assert "rope" not in got["launched"] and "blend_scatter" not in got["launched"]
    if T_max == 1 and flags == K.KVB_QKV_SPLIT_K and not cached and s.dtype == "bf16":
        # one row replacing nothing cached (decode): RoPE and the K/V store in the product's epilogue
        assert "rope_fuse" not in got["launched"] and got["launched"]["gemm_qkv"]["count"] == 1
    else:
        assert "rope_fuse" in got["launched"]
    for key in ("q", "k", "v", "kp", "vp", "alpha", "d", "ck"):
        assert torch.equal(got[key], ref[key]), key
    q, k, v, kp, vp, alpha, d_out, ck = (got[x] for x in ("q", "k", "v", "kp", "vp", "alpha", "d", "ck"))
    n = n_valid
    Wn = {kk: np64(vv) for kk, vv in W.items()}
    rq, rk, rv = OM.qkv(np64(hidden)[rows[:n]], pos[rows[:n]], Wn, s)
    tol = TOL[s.dtype]
    assert max_rel_err(q[:n], rq) < tol and max_rel_err(k[:n], rk) < tol and max_rel_err(v[:n], rv) < tol
    assert torch.all(q[n:] == 7.0) and torch.all(k[n:] == 7.0) and torch.all(v[n:] == 7.0)
    kr, vr = np64(k)[:n], np64(v)[:n]                 # the call's own recomputed rows
    reuse_k = _rows_at(kp0, src_slot[rows[:n]], s)
    reuse_v = _rows_at(vp0, src_slot[rows[:n]], s)
    ok = dst[:n] >= 0
    if cached:
        d_ref = OS.deviation(kr, reuse_k)
        a_new = OS.alpha_of(d_ref, OS.row_sq(reuse_k))
        a_use = {K.KVB_ALPHA_LAG: alpha0[rows[:n]].astype(np.float64), K.KVB_ALPHA_CURRENT: a_new,
                 K.KVB_ALPHA_ONE: np.ones(n)}[mode]
        kb = OM.store(OS.blend(a_use, kr, reuse_k), s.dtype)
        vb = OM.store(OS.blend(a_use, vr, reuse_v), s.dtype)
        assert np.allclose(np64(d_out)[:n], d_ref, rtol=2e-5, atol=1e-6) and np.all(np64(d_out)[n:] == -1.0)
        assert np.allclose(np64(ck)[:n], OS.cksim(kr, reuse_k), atol=2e-5)
        a_got = np64(alpha)
        if mode == K.KVB_ALPHA_ONE:
            assert np.array_equal(a_got, alpha0.astype(np.float64))
        else:
            assert np.allclose(a_got[rows[:n]], a_new, rtol=2e-5, atol=1e-7)
        if mode == K.KVB_ALPHA_LAG:    # alpha = 1: the recomputed row itself
            assert np.array_equal(_rows_at(kp, dst[:1], s), kr[:1])
    else:
        kb, vb = kr, vr
    assert max_rel_err(_rows_at(kp, dst[:n][ok], s), kb[ok]) < tol
    assert max_rel_err(_rows_at(vp, dst[:n][ok], s), vb[ok]) < tol
    if mode == K.KVB_ALPHA_ONE:
        assert np.array_equal(_rows_at(kp, dst[:n][ok], s), kr[ok])
    # nothing else in the pools moved
    touched = np.zeros(n_pages * 16, bool)
    touched[dst[:n][ok]] = True
    untouched = np.flatnonzero(~touched)
    assert np.array_equal(_rows_at(kp, untouched, s), _rows_at(kp0, untouched, s))
    assert np.array_equal(_rows_at(vp, untouched, s), _rows_at(vp0, untouched, s))


def test_qkv_fused_rows_are_batch_invariant(ctx):
    """With KVB_QKV_BATCH_INVARIANT a row's rotated q/k/v and its scattered K/V
    are bitwise the same whatever batch it sits in."""
    s = SHAPES["bf16"]
    g = np.random.default_rng(8)
    desc = K.model_desc(s)
    n_tok, n_pages = 400, 64
    hidden = rand((n_tok, s.d_model), g, dtype=torch.bfloat16).to(DEV)
    W = weights(s, g)
    pos = i32(g.integers(0, 5000, n_tok))
    outs = []
    for rows in (np.arange(0, 150), np.concatenate([np.arange(250, 400), np.arange(0, 150)])):
        T = len(rows)
        q = torch.empty((T, s.n_q_heads, s.head_dim), dtype=torch.bfloat16, device=DEV)
        k = torch.empty((T, s.n_kv_heads, s.head_dim), dtype=torch.bfloat16, device=DEV)
        v = torch.empty_like(k)
        kp = torch.zeros((n_pages, s.n_kv_heads, 16, s.head_dim), dtype=torch.bfloat16, device=DEV)
        vp = torch.zeros_like(kp)
        ws, wsb = workspace(ctx, desc, T, n_tok)
        K.kvb_qkv_fused(ctx, sh(), desc, T, None, i32(rows), hidden, W["norm1"], W["w_qkv"], pos, q, k, v, kp, vp,
                        n_pages, None, i32(rows), K.KVB_ALPHA_ONE, None, None, None, ws, wsb)
        outs.append((q, k, v, kp, vp))
    torch.cuda.synchronize()
    for a, b in zip(outs[0][:3], outs[1][:3]):
        assert torch.equal(a[:150], b[150:300])
    for a, b in zip(outs[0][3:], outs[1][3:]):   # the slots of tokens 0..149 (the second batch also wrote others)
        assert np.array_equal(_rows_at(a, np.arange(150), s), _rows_at(b, np.arange(150), s))


def test_blend_scatter_without_cache(ctx):
    s = SHAPES["bf16"]
    g = np.random.default_rng(2)
    desc = K.model_desc(s)
    kp, vp = _pool(s, 8, g)
    T = 100
    dst = g.permutation(128)[:T]
    k_rec = rand((T, s.n_kv_heads, s.head_dim), g, dtype=torch.bfloat16).to(DEV)
    v_rec = rand((T, s.n_kv_heads, s.head_dim), g, dtype=torch.bfloat16).to(DEV)
    K.kvb_blend_scatter(ctx, sh(), desc, T, None, None, k_rec, v_rec, kp, vp, 8, None, i32(dst), K.KVB_ALPHA_ONE,
                        None, None, None)
    torch.cuda.synchronize()
    assert np.array_equal(_rows_at(kp, dst, s), np64(k_rec))
    assert np.array_equal(_rows_at(vp, dst, s), np64(v_rec))


# ------------------------------------------------------------------ attention

def _attn_case(s, g, req_lens, n_sel, extra_pages=4):
    n_tok = sum(req_lens)
    cu = np.concatenate([[0], np.cumsum(req_lens)])
    lo = np.concatenate([np.full(n, cu[b]) for b, n in enumerate(req_lens)])
    n_pages = (n_tok + 15) // 16 + extra_pages
    slot_map = g.permutation(n_pages * 16)[:n_tok]
    rows = np.sort(g.choice(n_tok, n_sel, replace=False))
    return n_tok, lo, n_pages, slot_map, rows


@pytest.mark.parametrize("name", ["bf16", "bf16_hd64", "fp32"])
@pytest.mark.parametrize("req_lens,n_sel", [([700], 180), ([300, 517, 64], 240), ([33], 33), ([2500], 7)])
@pytest.mark.parametrize("split", [False, True], ids=["unsplit", "split"])
def test_sparse_query_attention(ctx, name, req_lens, n_sel, split):
    """With workspace, bf16 cuts each block's key range over several workgroups
    and merges their partial results (split-KV); without, one pass per block."""
    s = SHAPES[name]
    g = np.random.default_rng(sum(req_lens) + n_sel)
    desc = K.model_desc(s)
    dt = tdt(s)
    n_tok, lo, n_pages, slot_map, rows = _attn_case(s, g, req_lens, n_sel)
    kp, vp = _pool(s, n_pages, g)
    T_max = n_sel + 9
    n_valid = n_sel
    rows_dev = np.concatenate([rows, np.zeros(9, dtype=rows.dtype)])
    q = rand((T_max, s.n_q_heads, s.head_dim), g, 1.5, dtype=dt).to(DEV)
    o = torch.full((T_max, s.q_dim), 3.0, dtype=dt, device=DEV)
    ws, wsb = workspace(ctx, desc, T_max, n_tok) if split else (None, 0)
    if split:
        ws.fill_(0xFF)   # partial results must not depend on the workspace's previous contents
    K.kvb_timing_enable(ctx, "attention_merge")
    K.kvb_sparse_query_attn(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows_dev), i32(lo), q, kp, vp, n_pages,
                            i32(slot_map), 1.0 / np.sqrt(s.head_dim), o, ws, wsb)
    merged = K.kvb_timing_read(ctx).get("attention_merge", {}).get("count", 0)
    K.kvb_timing_enable(ctx, None)
    assert merged == (1 if split and s.dtype == "bf16" else 0)
    torch.cuda.synchronize()
    Klog, Vlog = _rows_at(kp, slot_map, s), _rows_at(vp, slot_map, s)
    ref = OM.attention_rows(np64(q)[:n_valid], rows, Klog, Vlog, lo[rows], s)
    assert max_rel_err(o[:n_valid], ref) < TOL[s.dtype]
    assert torch.all(o[n_valid:] == 3.0)


FEW_SHAPES = {
    "bf16": SHAPES["bf16"],                      # group of 4, head dim 128
    "bf16_hd64": SHAPES["bf16_hd64"],            # group of 8, head dim 64
    "bf16_g1": wl.ModelShape(n_layers=1, d_model=512, n_q_heads=4, n_kv_heads=4, head_dim=128, ffn=512,
                             dtype="bf16"),
    "bf16_g16": wl.ModelShape(n_layers=1, d_model=2048, n_q_heads=16, n_kv_heads=1, head_dim=128, ffn=512,
                              dtype="bf16"),
}


@pytest.mark.parametrize("name", list(FEW_SHAPES))
@pytest.mark.parametrize("req_lens,rows_at,T_max", [
    ([2500], [2499], 1),                   # one decode-like row over a long prompt
    ([2500], [1300], 2),                   # one valid row of two (the padding row stays untouched)
    ([300, 517, 64], [299, 816, 880], 3),  # one row per request, each at its request's end
    ([700], [0, 63, 64, 699], 4),          # rows at tile edges, including the first token
])
@pytest.mark.parametrize("split", [False, True], ids=["unsplit", "split"])
def test_few_rows_attention(ctx, name, req_lens, rows_at, T_max, split):
    """A handful of query rows (decode) runs the per-row kernel: one block per
    (row, KV head, key split); with workspace its splits go through the merge."""
    s = FEW_SHAPES[name]
    g = np.random.default_rng(sum(req_lens) + T_max + 17 * len(name))
    desc = K.model_desc(s)
    dt = tdt(s)
    n_tok = sum(req_lens)
    cu = np.concatenate([[0], np.cumsum(req_lens)])
    lo = np.concatenate([np.full(n, cu[b]) for b, n in enumerate(req_lens)])
    n_pages = (n_tok + 15) // 16 + 5
    slot_map = g.permutation(n_pages * 16)[:n_tok]
    rows = np.array(rows_at, dtype=np.int64)
    n_valid = len(rows)
    rows_dev = np.concatenate([rows, np.zeros(T_max - n_valid, dtype=rows.dtype)])
    kp, vp = _pool(s, n_pages, g)
    q = rand((T_max, s.n_q_heads, s.head_dim), g, 1.5, dtype=dt).to(DEV)
    o = torch.full((T_max, s.q_dim), 3.0, dtype=dt, device=DEV)
    ws, wsb = workspace(ctx, desc, T_max, n_tok) if split else (None, 0)
    if split:
        ws.fill_(0xFF)
    K.kvb_timing_enable(ctx, "attention")
    K.kvb_sparse_query_attn(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows_dev), i32(lo), q, kp, vp, n_pages,
                            i32(slot_map), 1.0 / np.sqrt(s.head_dim), o, ws, wsb)
    t = K.kvb_timing_read(ctx)
    K.kvb_timing_enable(ctx, None)
    assert t["attention"]["count"] == 1
    assert t.get("attention_merge", {}).get("count", 0) == (1 if split else 0)
    torch.cuda.synchronize()
    Klog, Vlog = _rows_at(kp, slot_map, s), _rows_at(vp, slot_map, s)
    ref = OM.attention_rows(np64(q)[:n_valid], rows, Klog, Vlog, lo[rows], s)
    assert max_rel_err(o[:n_valid], ref) < TOL[s.dtype]
    assert torch.all(o[n_valid:] == 3.0)


# ------------------------------------------------------------------ CacheBlend-style attention-map deviation

AMAP_SHAPES = {
    "bf16": SHAPES["bf16"],
    "bf16_hd64": SHAPES["bf16_hd64"],
    "bf16_g8": wl.ModelShape(n_layers=1, d_model=2048, n_q_heads=16, n_kv_heads=2, head_dim=128, ffn=512,
                             dtype="bf16"),
    "fp32": SHAPES["fp32"],
}


@pytest.mark.parametrize("name", list(AMAP_SHAPES))
@pytest.mark.parametrize("req_lens,invalid", [([700], False), ([300, 517, 64], False), ([33], False),
                                              ([300, 517, 64], True)])
def test_attnmap_deviation(ctx, name, req_lens, invalid):
    """dev vs the oracle; tokens whose visible cached keys equal the recomputed
    ones get exactly 0; a key with an invalid reuse slot is left out of both maps."""
    s = AMAP_SHAPES[name]
    g = np.random.default_rng(7 * sum(req_lens) + invalid)
    desc = K.model_desc(s)
    dt = tdt(s)
    B, n_tok = len(req_lens), sum(req_lens)
    cu = np.concatenate([[0], np.cumsum(req_lens)]).astype(np.int64)
    lo = np.concatenate([np.full(n, cu[b]) for b, n in enumerate(req_lens)])
    n_pages = (n_tok + 15) // 16 + 3
    reuse_slot = g.permutation(n_pages * 16)[:n_tok]
    k_rec = rand((n_tok, s.n_kv_heads, s.head_dim), g, dtype=dt)
    kp = rand((n_pages, s.n_kv_heads, 16, s.head_dim), g, dtype=dt)
    # cached keys: the recomputed ones for each request's first 40 tokens, a
    # perturbation of them (position-shift-like) elsewhere
    cached = k_rec.float() + 0.3 * rand((n_tok, s.n_kv_heads, s.head_dim), g)
    for b in range(B):
        cached[cu[b]:cu[b] + min(40, req_lens[b])] = k_rec[cu[b]:cu[b] + min(40, req_lens[b])].float()
    sl = torch.as_tensor(reuse_slot)
    kp[sl // 16, :, sl % 16, :] = cached.to(dt)
    if invalid:
        reuse_slot[cu[:-1]] = -5          # first key of every request: no valid slot
    q = rand((n_tok, s.n_q_heads, s.head_dim), g, 1.5, dtype=dt)
    q, k_rec, kp = q.to(DEV), k_rec.to(DEV), kp.to(DEV)
    dev = torch.full((n_tok,), -1.0, device=DEV)
    ws, wsb = workspace(ctx, desc, 1, n_tok, B)
    scale = 1.0 / np.sqrt(s.head_dim)
    K.kvb_attnmap_deviation(ctx, sh(), desc, n_tok, i32(lo), q, k_rec, kp, n_pages, i32(reuse_slot), scale, dev, ws,
                            wsb)
    torch.cuda.synchronize()
    got = np64(dev)
    reuse = _rows_at(kp, reuse_slot, s)
    idx = np.arange(n_tok)
    lo_ref = np.minimum(lo + 1, idx) if invalid else lo
    ref = OS.attention_map_deviation(np64(q), np64(k_rec), reuse, lo_ref, s)
    if invalid:
        ref[cu[:-1]] = 0.0
    # fp32 scores: absolute error of a probability ~ 1e-6 of its value, summed over a row
    assert np.allclose(got, ref, rtol=1e-3, atol=5e-5), np.max(np.abs(got - ref))
    for b in range(B):
        n0 = min(40, req_lens[b])
        assert np.all(got[cu[b]:cu[b] + n0] == 0.0)
    assert np.all(got[np.abs(ref) > 1e-3] > 0.0)


@pytest.mark.parametrize("req_lens", [[517], [4100, 300, 2049, 64], [2048, 2048]])
def test_topk_from_scores(ctx, req_lens):
    """kvb_topk on given scores (zeros and exact ties included) equals the
    oracle's ranking and top-k of the same scores, bit for bit."""
    s = SHAPES["bf16"]
    g = np.random.default_rng(len(req_lens))
    desc = K.model_desc(s)
    B, n_tok = len(req_lens), sum(req_lens)
    cu = np.concatenate([[0], np.cumsum(req_lens)]).astype(np.int64)
    d_np = g.random(n_tok).astype(np.float32) * 2.0
    d_np[g.random(n_tok) < 0.2] = 0.0
    d_np[g.choice(n_tok, n_tok // 10)] = np.float32(0.75)
    d = torch.tensor(d_np, device=DEV)
    k_cap = [int(np.floor(0.15 * n)) for n in req_lens]
    ranking = torch.full((n_tok,), -1, dtype=torch.int32, device=DEV)
    s_count = torch.zeros(B, dtype=torch.int32, device=DEV)
    sel = torch.full((n_tok,), -1, dtype=torch.int32, device=DEV)
    cu_rows = torch.zeros(B + 1, dtype=torch.int32, device=DEV)
    cursor = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws, wsb = workspace(ctx, desc, 1, n_tok, B)
    K.kvb_topk(ctx, sh(), desc, B, n_tok, i32(cu), d, i32(k_cap), ranking, s_count, sel, cu_rows, cursor, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(d.cpu(), torch.tensor(d_np))
    rk, ss, sl, cr, cs = (x.cpu().numpy() for x in (ranking, s_count, sel, cu_rows, cursor))
    assert cr[0] == 0
    for b in range(B):
        seg = d_np[cu[b]:cu[b + 1]].astype(np.float64)
        ranking_ref, S_k_ref, cur_ref = OS.top_k(seg, k_cap[b])
        assert ss[b] == len(ranking_ref)
        assert list(rk[cu[b]:cu[b] + len(ranking_ref)] - cu[b]) == ranking_ref
        assert cs[b] == cur_ref == cr[b + 1] - cr[b]
        assert list(sl[cr[b]:cr[b + 1]] - cu[b]) == S_k_ref


# ------------------------------------------------------------------ O-proj + MLP

@pytest.mark.parametrize("name", ["bf16", "bf16_wide", "bf16_ragged", "fp32"])
@pytest.mark.parametrize("T_max,n_valid", [(230, 201), (64, 64), (7, 5), (1, 1)])
def test_mlp(ctx, name, T_max, n_valid):
    """O-proj + MLP on gathered rows; the small batches take the 64-row tiles with split-K,
    a single row the one-row product."""
    s = SHAPES[name]
    g = np.random.default_rng(8 + T_max)
    desc = K.model_desc(s)
    dt = tdt(s)
    n_tok = 400
    hidden0 = rand((n_tok, s.d_model), g, dtype=dt)
    hidden = hidden0.to(DEV)
    W = weights(s, g)
    rows = np.sort(g.choice(n_tok, T_max, replace=False))
    o = rand((T_max, s.q_dim), g, dtype=dt).to(DEV)
    wsb = K.kvb_workspace_size(ctx, desc, T_max, n_tok, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    K.kvb_mlp(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows), o, W["w_o"], hidden, W["norm2"], W["w_gate_up"],
              W["w_down"], ws, wsb)
    torch.cuda.synchronize()
    Wn = {kk: np64(vv) for kk, vv in W.items()}
    r = rows[:n_valid]
    ref = OM.post_attention(np64(hidden0)[r], np64(o)[:n_valid], Wn, s)
    assert max_rel_err(hidden[r], ref) < TOL[s.dtype]
    others = np.setdiff1d(np.arange(n_tok), r)
    assert torch.equal(hidden[others].cpu(), hidden0[others])


@pytest.mark.parametrize("T_max", [700, 1000, 1300, 1700, 2500, 2800, 4200, 6300])
def test_gemm_tile_epilogues(ctx, T_max):
    """Q/K/V projection (batch-invariant and split-K launches), O-projection and
    MLP at row counts for which the launch rule on a 256-CU device picks, over
    the eight sizes, every tile shape's own epilogue (no split) in every mode:
    256x256, 192x256, 256x128 and 128x128 for Q/K/V, residual, SwiGLU and
    scatter, 64x256 for Q/K/V and SwiGLU.  Gathered rows, a row count below
    the launch bound, oracle on sampled rows (tile edges included), untouched
    rows checked whole."""
    s = SHAPES["bf16_wide"]
    g = np.random.default_rng(70 + T_max)
    desc = K.model_desc(s)
    dt = tdt(s)
    n_valid = T_max - 29
    n_tok = T_max + 97
    W = weights(s, g)
    Wn = {kk: np64(vv) for kk, vv in W.items()}
    hidden0 = rand((n_tok, s.d_model), g, dtype=dt)
    rows = np.sort(g.choice(n_tok, T_max, replace=False))
    pos = g.integers(0, 32768, n_tok)
    edges = [e + d_ for e in (64, 128, 192, 256, 384, 512, 768, 1024) for d_ in (-1, 0)]
    smp = np.unique(np.concatenate([[0, n_valid - 1], [e for e in edges if e < n_valid],
                                    g.choice(n_valid, 40, replace=False)]))
    ws, wsb = workspace(ctx, desc, T_max, n_tok)

    for flags in (K.KVB_QKV_BATCH_INVARIANT, K.KVB_QKV_SPLIT_K):
        hidden = hidden0.to(DEV)
        q = torch.full((T_max, s.n_q_heads, s.head_dim), 7.0, dtype=dt, device=DEV)
        k = torch.full((T_max, s.n_kv_heads, s.head_dim), 7.0, dtype=dt, device=DEV)
        v = torch.full((T_max, s.n_kv_heads, s.head_dim), 7.0, dtype=dt, device=DEV)
        K.kvb_qkv_proj(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows), hidden, W["norm1"], W["w_qkv"], i32(pos),
                       q, k, v, ws, wsb, flags)
        torch.cuda.synchronize()
        rq, rk, rv = OM.qkv(np64(hidden0)[rows[smp]], pos[rows[smp]], Wn, s)
        assert max_rel_err(q[smp], rq) < TOL[s.dtype]
        assert max_rel_err(k[smp], rk) < TOL[s.dtype]
        assert max_rel_err(v[smp], rv) < TOL[s.dtype]
        assert torch.all(q[n_valid:] == 7.0) and torch.all(k[n_valid:] == 7.0) and torch.all(v[n_valid:] == 7.0)

    hidden = hidden0.to(DEV)
    o = rand((T_max, s.q_dim), g, dtype=dt).to(DEV)
    K.kvb_mlp(ctx, sh(), desc, T_max, i32([n_valid]), i32(rows), o, W["w_o"], hidden, W["norm2"], W["w_gate_up"],
              W["w_down"], ws, wsb)
    torch.cuda.synchronize()
    ref = OM.post_attention(np64(hidden0)[rows[smp]], np64(o)[smp], Wn, s)
    assert max_rel_err(hidden[rows[smp]], ref) < TOL[s.dtype]
    others = np.setdiff1d(np.arange(n_tok), rows[:n_valid])
    assert torch.equal(hidden[others].cpu(), hidden0[others])


# ------------------------------------------------------------------ deviation + top-k

DEV_SHAPES = {
    "bf16": SHAPES["bf16"],            # one block per token (K/V row of 256 elements)
    "fp32": SHAPES["fp32"],
    "bf16_wide": SHAPES["bf16_wide"],  # 4 KV heads x 128: one wave per 4 tokens, one vector per lane
    "bf16_kv8": wl.ModelShape(n_layers=1, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=512,
                              dtype="bf16"),  # the Mistral rows: two vectors per lane
    "bf16_kv8_hd64": wl.ModelShape(n_layers=1, d_model=2048, n_q_heads=32, n_kv_heads=8, head_dim=64, ffn=512,
                                   dtype="bf16"),
}


@pytest.mark.parametrize("name,invalid", [(n, False) for n in DEV_SHAPES] + [("bf16", True), ("bf16_kv8", True)],
                         ids=[n for n in DEV_SHAPES] + ["bf16-invalid", "bf16_kv8-invalid"])
@pytest.mark.parametrize("req_lens", [[517], [4100, 300, 2049, 64], [2048, 2048]])
def test_deviation_topk(ctx, name, invalid, req_lens):
    """d, alpha vs the oracle; the top-k of the GPU's d bit-exact; with
    `invalid`, tokens whose reused slot lies outside the pool (one shape per
    kernel) are compared with a zero cached key."""
    s = DEV_SHAPES[name]
    g = np.random.default_rng(sum(req_lens))
    desc = K.model_desc(s)
    dt = tdt(s)
    B, n_tok = len(req_lens), sum(req_lens)
    cu = np.concatenate([[0], np.cumsum(req_lens)]).astype(np.int64)
    n_pages = (n_tok + 15) // 16 + 2
    kp, _ = _pool(s, n_pages, g)
    reuse_slot = g.permutation(n_pages * 16)[:n_tok]
    k_rec = rand((n_tok, s.n_kv_heads, s.head_dim), g, dtype=dt)
    reuse = _rows_at(kp, reuse_slot, s)
    # first chunk of every request reproduces the cache exactly (d = 0); some exact ties
    for b in range(B):
        n0 = min(40, req_lens[b])
        k_rec[cu[b]:cu[b] + n0] = torch.tensor(reuse[cu[b]:cu[b] + n0], dtype=torch.float32).to(dt)
    # exact ties: a few tokens share both their recomputed key and their cached slot
    for b in range(B):
        n = req_lens[b]
        if n > 60:
            for a, c in [(n - 1, n - 5), (n - 2, n - 9), (45, n - 3)]:
                reuse_slot[cu[b] + c] = reuse_slot[cu[b] + a]
                k_rec[cu[b] + c] = k_rec[cu[b] + a]
    reuse = _rows_at(kp, reuse_slot, s)
    if invalid:
        # three tokens per request without a cached row (negative, or past the pool's end)
        for b in range(B):
            for j, bad in [(req_lens[b] // 2, -1), (req_lens[b] - 1, n_pages * 16 + 5), (req_lens[b] // 3, -7)]:
                reuse_slot[cu[b] + j] = bad
                reuse[cu[b] + j] = 0.0
    k_rec = k_rec.to(DEV)
    k_cap = [int(np.floor(0.26 * n)) for n in req_lens]
    d = torch.zeros(n_tok, device=DEV)
    alpha = torch.zeros(n_tok, device=DEV)
    ranking = torch.full((n_tok,), -1, dtype=torch.int32, device=DEV)
    s_count = torch.zeros(B, dtype=torch.int32, device=DEV)
    sel = torch.full((n_tok,), -1, dtype=torch.int32, device=DEV)
    cu_rows = torch.zeros(B + 1, dtype=torch.int32, device=DEV)
    cursor = torch.zeros(B, dtype=torch.int32, device=DEV)
    wsb = K.kvb_workspace_size(ctx, desc, 1, n_tok, B)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    K.kvb_deviation_topk(ctx, sh(), desc, B, n_tok, i32(cu), k_rec, kp, n_pages, i32(reuse_slot), i32(k_cap), d,
                         alpha, ranking, s_count, sel, cu_rows, cursor, ws, wsb)
    torch.cuda.synchronize()
    d_ref = OS.deviation(np64(k_rec), reuse)
    gd = np64(d)
    assert np.allclose(gd, d_ref, rtol=2e-5, atol=0)
    assert np.allclose(np64(alpha), OS.alpha_of(d_ref, OS.row_sq(reuse)), rtol=2e-5, atol=1e-7)
    rk, ss, sl, cr, cs = (x.cpu().numpy() for x in (ranking, s_count, sel, cu_rows, cursor))
    off = 0
    assert cr[0] == 0
    for b in range(B):
        seg = gd[cu[b]:cu[b + 1]]
        ranking_ref, S_k_ref, cur_ref = OS.top_k(seg, k_cap[b])   # exact top-k of the GPU's own d
        nS = len(ranking_ref)
        assert ss[b] == nS
        assert list(rk[cu[b]:cu[b] + nS] - cu[b]) == ranking_ref
        zeros = sorted(set(range(req_lens[b])) - set(ranking_ref))
        assert list(rk[cu[b] + nS:cu[b + 1]] - cu[b]) == zeros
        assert cs[b] == cur_ref == cr[b + 1] - cr[b]
        assert list(sl[cr[b]:cr[b + 1]] - cu[b]) == S_k_ref
        # against the oracle's own float64 d: equal except inside the 1e-3 band around the k-th value
        _, S_oracle, _ = OS.top_k(d_ref[cu[b]:cu[b + 1]], k_cap[b])
        diff = set(S_oracle) ^ set(S_k_ref)
        if diff:
            kth = np.sort(d_ref[cu[b]:cu[b + 1]])[::-1][len(S_oracle) - 1]
            for i in diff:
                assert abs(d_ref[cu[b] + i] - kth) <= 1e-3 * kth
        off += cur_ref


# ------------------------------------------------------------------ refresh

@pytest.mark.parametrize("rule", [K.KVB_REFRESH_LITERAL, K.KVB_REFRESH_DISSIM])
def test_cosine_refresh(ctx, rule):
    s = SHAPES["bf16"]
    g = np.random.default_rng(40 + rule)
    desc = K.model_desc(s)
    req_lens = [3000, 700, 1500, 90]
    B, n_tok = len(req_lens), sum(req_lens)
    cu = np.concatenate([[0], np.cumsum(req_lens)])
    tau = float(np.float32(0.12))
    rankings, sels, curs, scount, cks = [], [], [], [], []
    for b, n in enumerate(req_lens):
        nS = int(n * g.uniform(0.3, 0.95))
        rk = list(g.permutation(n)[:nS])
        k = int(0.26 * n)
        cur = min(k + int(g.integers(0, 50)), nS)
        if b == 3:
            cur = nS - 2                                   # ranking nearly exhausted
        S_k = sorted(rk[:cur][-k:]) if cur else []
        rankings.append(rk)
        sels.append(S_k)
        curs.append(cur)
        scount.append(nS)
        cks.append(g.uniform(-0.2, 1.0, len(S_k)).astype(np.float32))
    ranking = np.zeros(n_tok, np.int64)
    for b in range(B):
        ranking[cu[b]:cu[b] + len(rankings[b])] = np.asarray(rankings[b]) + cu[b]
    sel_in = np.concatenate([np.asarray(x, np.int64) + cu[b] for b, x in enumerate(sels)])
    cu_in = np.concatenate([[0], np.cumsum([len(x) for x in sels])])
    T = len(sel_in)
    cursor = i32(curs)
    sel_out = torch.full((n_tok,), -1, dtype=torch.int32, device=DEV)
    cu_out = torch.zeros(B + 1, dtype=torch.int32, device=DEV)
    wsb = K.kvb_workspace_size(ctx, desc, 1, n_tok, B)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    K.kvb_cosine_refresh(ctx, sh(), desc, B, n_tok, i32(cu), T, i32(cu_in), i32(sel_in),
                         torch.tensor(np.concatenate(cks), device=DEV), tau, rule, i32(ranking), i32(scount), cursor,
                         sel_out, cu_out, ws, wsb)
    torch.cuda.synchronize()
    so, co, cur_o = sel_out.cpu().numpy(), cu_out.cpu().numpy(), cursor.cpu().numpy()
    rname = "literal" if rule == K.KVB_REFRESH_LITERAL else "dissim"
    assert co[0] == 0
    for b in range(B):
        exp_S, exp_cur, _ = OS.refresh(sels[b], cks[b].astype(np.float64), tau, rankings[b], curs[b], rname)
        assert list(so[co[b]:co[b + 1]] - cu[b]) == exp_S
        assert cur_o[b] == exp_cur


# ------------------------------------------------------------------ slot maps, embedding

def test_slot_map(ctx):
    s = SHAPES["bf16"]
    g = np.random.default_rng(4)
    desc = K.model_desc(s)
    req_lens = [500, 77, 300]
    B, n_tok = 3, 877
    cu = np.concatenate([[0], np.cumsum(req_lens)])
    reuse = g.permutation(5000)[:n_tok]
    sels = [np.sort(g.choice(n, k, replace=False)) + cu[b] for b, (n, k) in enumerate(zip(req_lens, [130, 20, 78]))]
    caps = [130, 20, 60]                 # request 2 has fewer new pages than selected rows
    pages = [list(g.permutation(np.arange(400, 600))[: (c + 15) // 16]) for c in caps]
    sel = np.concatenate(sels)
    cu_rows = np.concatenate([[0], np.cumsum([len(x) for x in sels])])
    T = len(sel)
    slot_map = torch.zeros(n_tok, dtype=torch.int32, device=DEV)
    dst = torch.zeros(T, dtype=torch.int32, device=DEV)
    n_pages = 600
    dirty = torch.zeros(n_pages, dtype=torch.int32, device=DEV)
    dirty[405] = 7           # counters accumulate over calls
    K.kvb_slot_map(ctx, sh(), desc, B, n_tok, T, i32(cu_rows), i32(sel), i32(reuse),
                   i32(np.concatenate(pages)), i32(np.concatenate([[0], np.cumsum([len(p) for p in pages])])),
                   slot_map, dst, n_pages, dirty)
    torch.cuda.synchronize()
    sm, ds = slot_map.cpu().numpy(), dst.cpu().numpy()
    exp = reuse.astype(np.int64).copy()
    for b in range(B):
        n_ok = min(len(sels[b]), len(pages[b]) * 16)
        exp = OP.slot_map(exp, sels[b][:n_ok], pages[b])
        got = ds[cu_rows[b]:cu_rows[b + 1]]
        assert list(got[:n_ok]) == list(OP.slot_of(pages[b], np.arange(n_ok)))
        assert np.all(got[n_ok:] == -1)
    assert np.array_equal(sm, exp)
    # dirty counters: every selected token routed to a new page, layer-2 style
    routes = [(np.zeros(n_tok, dtype=np.int64), np.zeros(0, dtype=np.int64)), (exp, np.concatenate(
        [sels[b][:min(len(sels[b]), len(pages[b]) * 16)] for b in range(B)]))]
    want = OP.dirty_counts(n_pages, routes)
    want[405] += 7
    assert np.array_equal(dirty.cpu().numpy(), want)


def test_page_dirty_add(ctx):
    """Decode-style counter updates: slots past the row count, negative or past
    the pool are ignored; repeated pages accumulate."""
    desc = K.model_desc(SHAPES["bf16"])
    g = np.random.default_rng(9)
    n_pages = 50
    slots = g.integers(-20, n_pages * 16 + 40, size=700).astype(np.int32)
    slots[:100] = g.integers(0, 32, size=100)        # many hits on pages 0 and 1
    dirty = torch.zeros(n_pages, dtype=torch.int32, device=DEV)
    K.kvb_page_dirty_add(ctx, sh(), desc, 700, i32([650]), i32(slots), n_pages, dirty)
    torch.cuda.synchronize()
    ok = slots[:650][(slots[:650] >= 0) & (slots[:650] < n_pages * 16)]
    assert np.array_equal(dirty.cpu().numpy(), OP.dirty_counts(n_pages, [], ok))


def test_embed(ctx):
    s = SHAPES["bf16"]
    g = np.random.default_rng(9)
    desc = K.model_desc(s)
    table = rand((1000, s.d_model), g, dtype=torch.bfloat16).to(DEV)
    toks = g.integers(0, 1000, 300)
    toks[17] = 5000                                       # out of range: row skipped
    rows = np.sort(g.choice(300, 120, replace=False))
    hidden = torch.zeros((300, s.d_model), dtype=torch.bfloat16, device=DEV)
    K.kvb_embed(ctx, sh(), desc, 120, None, i32(rows), i32(toks), 1000, table, hidden)
    torch.cuda.synchronize()
    exp = np.zeros((300, s.d_model))
    ok = rows[toks[rows] < 1000]
    exp[ok] = np64(table)[toks[ok]]
    assert np.array_equal(np64(hidden), exp)
