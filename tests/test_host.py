"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, validates arguments before touching the
device, and its page allocator follows the documented deterministic rule."""
import ctypes
import os
import re

import numpy as np
import pytest

from selective_kv_cache_amd import _lib as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvb.h")


def header_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:kvb_status|const char\*)\s+(kvb_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        pytest.fail("libkvb.so is not built (python -m selective_kv_cache_amd.build)")
    return K.load()


def test_exports_every_header_symbol(lib):
    syms = header_symbols()
    assert len(syms) >= 19
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(K.EXPORTS)


def test_status_strings(lib):
    assert K.kvb_status_string(0) == "ok"
    assert "exhausted" in K.kvb_status_string(K.KVB_ERR_CAPACITY)
    assert "workspace" in K.kvb_status_string(K.KVB_ERR_WORKSPACE)


def test_pool_lowest_first_and_capacity(lib):
    p = K.kvb_pool_create(10)
    try:
        assert K.kvb_pool_alloc(p, 3) == [0, 1, 2]
        assert K.kvb_pool_alloc(p, 2) == [3, 4]
        K.kvb_pool_release(p, [1, 3])
        assert K.kvb_pool_free_count(p) == 7
        assert K.kvb_pool_alloc(p, 3) == [1, 3, 5]
        with pytest.raises(K.KvbError) as e:
            K.kvb_pool_alloc(p, 5)
        assert e.value.status == K.KVB_ERR_CAPACITY
        assert K.kvb_pool_free_count(p) == 4          # failed call allocated nothing
        with pytest.raises(K.KvbError) as e:
            K.kvb_pool_release(p, [9])
        assert e.value.status == K.KVB_ERR_INVALID_ARG
        assert K.kvb_pool_alloc(p, 0) == []
    finally:
        K.kvb_pool_destroy(p)


def test_pool_matches_worked_page_plan(lib):
    """The library allocator reproduces the hand-worked page plan of the tiny workload."""
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_tiny.json")))
    p = K.kvb_pool_create(4096)
    try:
        for uid, n in enumerate(g["chunk_lens"]):
            for l in range(2):
                assert K.kvb_pool_alloc(p, (n + 15) // 16) == g["compile_pages"][str(uid)][l]
        assert K.kvb_pool_alloc(p, 32) == g["link_pages"][0]
        assert K.kvb_pool_alloc(p, (133 + 15) // 16) == g["link_pages"][1]
    finally:
        K.kvb_pool_destroy(p)


def _desc(**kw):
    base = dict(d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688, page_size=16,
                rope_base=10000.0, rms_eps=1e-5, dtype=K.KVB_F32)
    base.update(kw)
    return K.kvb_model_desc(**base)


FAKE_CTX = ctypes.c_void_p(ctypes.addressof(ctypes.create_string_buffer(64)))


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), K.KVB_ERR_UNSUPPORTED),
    (dict(page_size=32), K.KVB_ERR_UNSUPPORTED),
    (dict(dtype=7), K.KVB_ERR_UNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=4), K.KVB_ERR_INVALID_ARG),
    (dict(d_model=0), K.KVB_ERR_INVALID_ARG),
    (dict(dtype=K.KVB_BF16, ffn=688), K.KVB_ERR_UNSUPPORTED),
])
def test_desc_validation(lib, kw, status):
    with pytest.raises(K.KvbError) as e:
        K.kvb_workspace_size(FAKE_CTX, _desc(**kw), 16, 16, 1)
    assert e.value.status == status
    assert K.kvb_last_error() != ""


def test_null_and_size_checks_enqueue_nothing(lib):
    d = _desc()
    with pytest.raises(K.KvbError) as e:
        K.kvb_qkv_proj(None, None, d, 4, None, None, 1, 1, 1, None, 1, 1, 1)
    assert e.value.status == K.KVB_ERR_INVALID_ARG
    with pytest.raises(K.KvbError) as e:
        K.kvb_qkv_proj(FAKE_CTX, None, d, 4, None, None, None, 1, 1, None, 1, 1, 1)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "hidden" in K.kvb_last_error()
    with pytest.raises(K.KvbError) as e:
        K.kvb_mlp(FAKE_CTX, None, d, 4, None, None, 1, 1, 1, 1, 1, 1, 1, 10)
    assert e.value.status == K.KVB_ERR_WORKSPACE
    with pytest.raises(K.KvbError) as e:
        K.kvb_blend_scatter(FAKE_CTX, None, d, 4, None, None, 1, 1, 1, 1, 8, None, 1, K.KVB_ALPHA_LAG, 1, None, None)
    assert e.value.status == K.KVB_ERR_INVALID_ARG
    with pytest.raises(K.KvbError) as e:
        K.kvb_cosine_refresh(FAKE_CTX, None, d, 1, 16, 1, 4, 1, 5, 1, 0.12, K.KVB_REFRESH_LITERAL, 1, 1, 1, 5, 1, 1,
                             1 << 20)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "overlap" in K.kvb_last_error()
    with pytest.raises(K.KvbError) as e:
        K.kvb_deviation_topk(FAKE_CTX, None, d, 1, 16, 1, 1, 1, 4, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 8)
    assert e.value.status == K.KVB_ERR_WORKSPACE
    with pytest.raises(K.KvbError) as e:  # bf16 normalises into the workspace
        K.kvb_qkv_proj(FAKE_CTX, None, _desc(dtype=K.KVB_BF16, d_model=512, ffn=1536, n_q_heads=8, head_dim=128),
                       4, None, None, 1, 1, 1, None, 1, 1, 1, None, 0)
    assert e.value.status == K.KVB_ERR_WORKSPACE
    # zero-size calls are valid no-ops
    K.kvb_qkv_proj(FAKE_CTX, None, d, 0, None, None, None, None, None, None, None, None, None)
    with pytest.raises(K.KvbError) as e:  # unknown flags
        K.kvb_qkv_proj(FAKE_CTX, None, d, 4, None, None, 1, 1, 1, None, 1, 1, 1, None, 0, 2)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "flags" in K.kvb_last_error()
    K.kvb_mlp(FAKE_CTX, None, d, 0, None, None, None, None, None, None, None, None, None, 0)


def test_workspace_size_monotone(lib):
    d = _desc(dtype=K.KVB_BF16, d_model=512, ffn=1536, n_q_heads=8, head_dim=128)
    a = K.kvb_workspace_size(FAKE_CTX, d, 100, 1000, 1)
    b = K.kvb_workspace_size(FAKE_CTX, d, 200, 1000, 1)
    c = K.kvb_workspace_size(FAKE_CTX, d, 200, 100000, 4)
    assert 0 < a <= b <= c
    assert b >= 200 * (512 + 1536) * 2


def test_product_code_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "selective_kv_cache_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "workloads" not in src or f.endswith(".py") is False or "import workloads" not in src, f


def test_pages_copy_checks(lib):
    """kvb_pages_copy: argument errors are reported before anything is enqueued."""
    d = _desc()
    for direction, ids, status in ((7, [0], K.KVB_ERR_INVALID_ARG), (K.KVB_COPY_H2D, [3, -1], K.KVB_ERR_INVALID_ARG)):
        with pytest.raises(K.KvbError) as e:
            K.kvb_pages_copy(FAKE_CTX, None, d, direction, 1, 1, 1, 1, ids)
        assert e.value.status == status
    with pytest.raises(K.KvbError) as e:
        K.kvb_pages_copy(None, None, d, K.KVB_COPY_H2D, 1, 1, 1, 1, [0])
    assert e.value.status == K.KVB_ERR_INVALID_ARG
    with pytest.raises(K.KvbError) as e:  # a destination without its source
        K.kvb_pages_copy(FAKE_CTX, None, d, K.KVB_COPY_H2D, None, 1, 1, 1, [0])
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "src_k" in K.kvb_last_error()
    K.kvb_pages_copy(FAKE_CTX, None, d, K.KVB_COPY_D2H, None, None, None, None, [])  # nothing to copy


def test_attnmap_and_topk_checks(lib):
    """kvb_attnmap_deviation / kvb_topk: argument errors before anything is enqueued."""
    d = _desc()
    bf = _desc(dtype=K.KVB_BF16, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536)
    with pytest.raises(K.KvbError) as e:          # no queries
        K.kvb_attnmap_deviation(FAKE_CTX, None, d, 8, 1, None, 1, 1, 4, 1, 0.125, 1, None, 0)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "q" in K.kvb_last_error()
    with pytest.raises(K.KvbError) as e:          # bf16 needs its partials workspace
        K.kvb_attnmap_deviation(FAKE_CTX, None, bf, 8, 1, 1, 1, 1, 4, 1, 0.125, 1, 1, 16)
    assert e.value.status == K.KVB_ERR_WORKSPACE
    g3 = _desc(dtype=K.KVB_BF16, d_model=768, n_q_heads=6, n_kv_heads=2, head_dim=128, ffn=1536)
    with pytest.raises(K.KvbError) as e:          # a GQA group of 3 does not tile the lanes
        K.kvb_attnmap_deviation(FAKE_CTX, None, g3, 8, 1, 1, 1, 1, 4, 1, 0.125, 1, 1, 1 << 20)
    assert e.value.status == K.KVB_ERR_UNSUPPORTED
    K.kvb_attnmap_deviation(FAKE_CTX, None, d, 0, None, None, None, None, 0, None, 0.125, None, None, 0)
    with pytest.raises(K.KvbError) as e:
        K.kvb_topk(FAKE_CTX, None, d, 0, 8, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1 << 20)
    assert e.value.status == K.KVB_ERR_INVALID_ARG
    with pytest.raises(K.KvbError) as e:
        K.kvb_topk(FAKE_CTX, None, d, 1, 8, 1, None, 1, 1, 1, 1, 1, 1, 1, 1 << 20)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "d" in K.kvb_last_error()
    with pytest.raises(K.KvbError) as e:
        K.kvb_topk(FAKE_CTX, None, d, 1, 8, 1, 1, 1, 1, 1, 1, 1, 1, 1, 8)
    assert e.value.status == K.KVB_ERR_WORKSPACE


def test_host_spill_order_matches_oracle(rng):
    from oracle import pages as OP
    from selective_kv_cache_amd.link import spill_order
    for _ in range(50):
        n = int(rng.integers(1, 40))
        counts = rng.integers(0, 4, n) * (rng.random(n) > 0.4)
        pages = rng.choice(n, int(rng.integers(0, n + 1)), replace=False)
        assert spill_order(counts, pages) == OP.spill_order(counts, pages)


LINK_FIELDS = [f for f, _ in K.kvb_link_desc._fields_]


def test_link_desc_layout_matches_header(tmp_path):
    """The ctypes kvb_link_desc and kvb_layer_weights have the C structs' size and offsets."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f if f not in ("sel", "cu_rows") else f + "[1]" for f in LINK_FIELDS]
    lines = [f'  printf("%zu\\n", offsetof(kvb_link_desc, {f}));' for f in fields]
    lines += ['  printf("%zu\\n", sizeof(kvb_link_desc));', '  printf("%zu\\n", sizeof(kvb_layer_weights));',
              '  printf("%zu\\n", offsetof(kvb_layer_weights, w_down));']
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kvb.h"\nint main(void) {\n'
                   + "\n".join(lines) + "\n  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [getattr(K.kvb_link_desc, f).offset + (8 if f in ("sel", "cu_rows") else 0) for f in LINK_FIELDS]
    want += [ctypes.sizeof(K.kvb_link_desc), ctypes.sizeof(K.kvb_layer_weights), K.kvb_layer_weights.w_down.offset]
    assert got == want


def test_link_run_checks(lib):
    """kvb_link_run refuses a missing or inconsistent description before queuing anything."""
    d = _desc()
    with pytest.raises(K.KvbError) as e:
        K._call("kvb_link_run", FAKE_CTX, None, d, None, None)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "link" in K.kvb_last_error()
    k = K.kvb_link_desc()
    k.mode, k.B, k.n_tok, k.n_layers, k.n_pages, k.vocab, k.rows, k.period = 0, 1, 64, 2, 8, 100, 16, 4
    with pytest.raises(K.KvbError) as e:
        K.kvb_link_run(FAKE_CTX, None, d, k)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "layers" in K.kvb_last_error()
    lw = (K.kvb_layer_weights * 2)(K.kvb_layer_weights(1, 1, 1, 1, 1, 1), K.kvb_layer_weights(1, 1, 1, 1, 1, None))
    k.layers = ctypes.addressof(lw)
    with pytest.raises(K.KvbError) as e:
        K.kvb_link_run(FAKE_CTX, None, d, k)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "layer 2" in K.kvb_last_error()
    lw[1] = K.kvb_layer_weights(1, 1, 1, 1, 1, 1)
    pages = (ctypes.c_void_p * 2)(1, 1)
    k.new_pages = k.cu_pages = ctypes.addressof(pages)
    for f in ("embedding", "tokens", "pos", "lo", "cu_tok", "k_cap", "reuse_slot", "page_table", "k_pool",
              "v_pool", "hidden", "q", "k", "v", "o", "d", "alpha", "dev", "cksim", "ranking", "s_count", "cursor",
              "dst_slot"):
        setattr(k, f, 1)
    k.sel[0], k.sel[1], k.cu_rows[0], k.cu_rows[1] = 1, 1, 2, 3
    with pytest.raises(K.KvbError) as e:  # one selection buffer for both
        K.kvb_link_run(FAKE_CTX, None, d, k)
    assert e.value.status == K.KVB_ERR_INVALID_ARG and "differ" in K.kvb_last_error()
    k.sel[1] = 5
    for bad in (dict(mode=3), dict(rows=65), dict(period=0), dict(refresh_rule=4), dict(alpha_mode=9)):
        k2 = K.kvb_link_desc.from_buffer_copy(k)
        for f, v in bad.items():
            setattr(k2, f, v)
        with pytest.raises(K.KvbError) as e:
            K.kvb_link_run(FAKE_CTX, None, d, k2)
        assert e.value.status == K.KVB_ERR_INVALID_ARG, bad
    with pytest.raises(K.KvbError) as e:  # everything set but the workspace
        K.kvb_link_run(FAKE_CTX, None, d, k)
    assert e.value.status == K.KVB_ERR_WORKSPACE
