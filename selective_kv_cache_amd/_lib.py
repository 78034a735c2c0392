"""ctypes binding of libkvb.so: the C ABI declared in include/kvb.h, same names.

Argument marshalling only.  Tensors are passed as raw device pointers
(`tensor.data_ptr()`), None becomes NULL, the stream is a HIP stream handle.
Every call raises KvbError when the library returns a status < 0.  Nothing
here computes any step of the method, and there is no fallback: without the
built library every call fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvb.so")

KVB_OK = 0
KVB_ERR_INVALID_ARG = -1
KVB_ERR_UNSUPPORTED = -2
KVB_ERR_HIP = -3
KVB_ERR_CAPACITY = -4
KVB_ERR_WORKSPACE = -5
KVB_F32, KVB_BF16 = 0, 1
KVB_ALPHA_LAG, KVB_ALPHA_CURRENT, KVB_ALPHA_ONE = 0, 1, 2
KVB_REFRESH_LITERAL, KVB_REFRESH_DISSIM = 0, 1
KVB_COPY_H2D, KVB_COPY_D2H = 0, 1
KVB_QKV_BATCH_INVARIANT, KVB_QKV_SPLIT_K = 0, 1
KVB_NOALLOC_MAX_TOKENS, KVB_NOALLOC_MAX_REQUESTS = 131072, 4096
KVB_LINK_CACHESLIDE, KVB_LINK_STATIC, KVB_LINK_CACHEBLEND = 0, 1, 2


class KvbError(RuntimeError):
    def __init__(self, name: str, status: int, msg: str):
        super().__init__(f"{name}: {msg} (status {status})")
        self.status = status


class kvb_model_desc(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn", c_int32), ("page_size", c_int32),
                ("rope_base", c_float), ("rms_eps", c_float), ("dtype", c_int32)]


class kvb_layer_weights(ctypes.Structure):
    _fields_ = [("norm1", c_void_p), ("w_qkv", c_void_p), ("w_o", c_void_p), ("norm2", c_void_p),
                ("w_gate_up", c_void_p), ("w_down", c_void_p)]


class kvb_link_desc(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("B", c_int32), ("n_tok", c_int32), ("n_layers", c_int32),
                ("n_pages", c_int32), ("vocab", c_int32), ("rows", c_int32), ("period", c_int32),
                ("refresh_rule", c_int32), ("alpha_mode", c_int32), ("tau", c_float), ("scale", c_float),
                ("layers", c_void_p), ("embedding", c_void_p), ("tokens", c_void_p), ("pos", c_void_p),
                ("lo", c_void_p), ("cu_tok", c_void_p), ("k_cap", c_void_p), ("reuse_slot", c_void_p),
                ("new_pages", c_void_p), ("cu_pages", c_void_p), ("static_rows", c_void_p),
                ("static_cu", c_void_p), ("page_table", c_void_p), ("k_pool", c_void_p), ("v_pool", c_void_p),
                ("hidden", c_void_p), ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("o", c_void_p),
                ("d", c_void_p), ("alpha", c_void_p), ("dev", c_void_p), ("cksim", c_void_p),
                ("ranking", c_void_p), ("s_count", c_void_p), ("cursor", c_void_p), ("sel", c_void_p * 2),
                ("cu_rows", c_void_p * 2), ("dst_slot", c_void_p), ("page_dirty", c_void_p), ("ws", c_void_p),
                ("ws_bytes", c_size_t)]


P = c_void_p
I = c_int32
_SIGS = {
    "kvb_status_string": ([I], ctypes.c_char_p),
    "kvb_last_error": ([], ctypes.c_char_p),
    "kvb_create": ([I, POINTER(c_void_p)], I),
    "kvb_destroy": ([P], I),
    "kvb_workspace_size": ([P, P, I, I, I, POINTER(c_size_t)], I),
    "kvb_timing_enable": ([P, ctypes.c_char_p], I),
    "kvb_timing_read": ([P, ctypes.c_char_p, c_size_t, POINTER(c_size_t)], I),
    "kvb_pool_create": ([I, POINTER(c_void_p)], I),
    "kvb_pool_destroy": ([P], I),
    "kvb_pool_alloc": ([P, I, P], I),
    "kvb_pool_release": ([P, I, P], I),
    "kvb_pool_free_count": ([P, POINTER(c_int32)], I),
    "kvb_pages_copy": ([P, P, P, I, P, P, P, P, P, I], I),
    "kvb_embed": ([P, P, P, I, P, P, P, I, P, P], I),
    "kvb_qkv_proj": ([P, P, P, I, P, P, P, P, P, P, P, P, P, P, c_size_t, I], I),
    "kvb_qkv_fused": ([P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, I, P, P, I, P, P, P, P, c_size_t, I], I),
    "kvb_rope": ([P, P, P, I, P, P, P, P, P], I),
    "kvb_blend_scatter": ([P, P, P, I, P, P, P, P, P, P, I, P, P, I, P, P, P], I),
    "kvb_sparse_query_attn": ([P, P, P, I, P, P, P, P, P, P, I, P, c_float, P, P, c_size_t], I),
    "kvb_mlp": ([P, P, P, I, P, P, P, P, P, P, P, P, P, c_size_t], I),
    "kvb_deviation_topk": ([P, P, P, I, I, P, P, P, I, P, P, P, P, P, P, P, P, P, P, c_size_t], I),
    "kvb_deviation_topk_noalloc": ([P, P, P, I, I, P, P, P, I, P, P, P, P, P, P, P, P, P], I),
    "kvb_topk": ([P, P, P, I, I, P, P, P, P, P, P, P, P, P, c_size_t], I),
    "kvb_attnmap_deviation": ([P, P, P, I, P, P, P, P, I, P, c_float, P, P, c_size_t], I),
    "kvb_cosine_refresh": ([P, P, P, I, I, P, I, P, P, P, c_float, I, P, P, P, P, P, P, c_size_t], I),
    "kvb_slot_map": ([P, P, P, I, I, I, P, P, P, P, P, P, P, I, P], I),
    "kvb_page_dirty_add": ([P, P, P, I, P, P, I, P], I),
    "kvb_link_run": ([P, P, P, P, P], I),
}
EXPORTS = tuple(_SIGS)

_lib = None


def load():
    """Load libkvb.so (once); raises KvbError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KvbError("load", KVB_ERR_HIP,
                           f"{LIB_PATH} is missing: build it with `python -m selective_kv_cache_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, ctypes.Structure):
        return ctypes.addressof(x)
    if isinstance(x, c_void_p):
        return x.value
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _check(name: str, status: int):
    if status != KVB_OK:
        lib = load()
        raise KvbError(name, status, f"{lib.kvb_status_string(status).decode()}: {lib.kvb_last_error().decode()}")


def _call(name, *args):
    f = getattr(load(), name)
    conv = []
    for a, t in zip(args, f.argtypes):
        if t is P:
            conv.append(_ptr(a))
        else:
            conv.append(a)
    _check(name, f(*conv))


def stream_handle(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def model_desc(shape) -> kvb_model_desc:
    return kvb_model_desc(shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                          shape.page_size, float(shape.rope_base), float(shape.rms_eps),
                          KVB_BF16 if shape.dtype == "bf16" else KVB_F32)


# ------------------------------------------------------------------ basics

def kvb_status_string(s: int) -> str:
    return load().kvb_status_string(s).decode()


def kvb_last_error() -> str:
    return load().kvb_last_error().decode()


def kvb_create(device: int = 0) -> c_void_p:
    out = c_void_p()
    _check("kvb_create", load().kvb_create(device, ctypes.byref(out)))
    return out


def kvb_destroy(ctx) -> None:
    _check("kvb_destroy", load().kvb_destroy(ctx))


def kvb_workspace_size(ctx, desc, max_rows: int, max_tokens: int, max_requests: int) -> int:
    out = c_size_t()
    _check("kvb_workspace_size", load().kvb_workspace_size(ctx, ctypes.addressof(desc), max_rows, max_tokens,
                                                           max_requests, ctypes.byref(out)))
    return out.value


def kvb_timing_enable(ctx, filter_) -> None:
    """filter_: None = off, "" = every kernel, else a substring of kernel names."""
    _check("kvb_timing_enable", load().kvb_timing_enable(ctx, None if filter_ is None else filter_.encode()))


def kvb_timing_read(ctx) -> dict:
    """Per-kernel {"name": {"count", "ms"}} since the last read (synchronises on the events)."""
    import json
    need = c_size_t()
    _check("kvb_timing_read", load().kvb_timing_read(ctx, None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(max(need.value, 2))
    _check("kvb_timing_read", load().kvb_timing_read(ctx, buf, len(buf), ctypes.byref(need)))
    return json.loads(buf.value.decode() or "{}")


def kvb_pool_create(n_pages: int) -> c_void_p:
    out = c_void_p()
    _check("kvb_pool_create", load().kvb_pool_create(n_pages, ctypes.byref(out)))
    return out


def kvb_pool_destroy(pool) -> None:
    _check("kvb_pool_destroy", load().kvb_pool_destroy(pool))


def kvb_pool_alloc(pool, n: int) -> list:
    buf = (c_int32 * max(n, 1))()
    _check("kvb_pool_alloc", load().kvb_pool_alloc(pool, n, buf))
    return list(buf[:n])


def kvb_pool_release(pool, ids) -> None:
    ids = list(ids)
    buf = (c_int32 * max(len(ids), 1))(*ids)
    _check("kvb_pool_release", load().kvb_pool_release(pool, len(ids), buf))


def kvb_pool_free_count(pool) -> int:
    out = c_int32()
    _check("kvb_pool_free_count", load().kvb_pool_free_count(pool, ctypes.byref(out)))
    return out.value


def kvb_pages_copy(ctx, stream, desc, direction, src_k, src_v, dst_k, dst_v, page_ids) -> None:
    """page_ids: host sequence of page ids (marshalled to a host int32 array)."""
    ids = [int(x) for x in page_ids]
    buf = (c_int32 * max(len(ids), 1))(*ids)
    _call("kvb_pages_copy", ctx, stream, desc, direction, src_k, src_v, dst_k, dst_v,
          ctypes.cast(buf, c_void_p).value, len(ids))


# ------------------------------------------------------------------ the path

def kvb_embed(ctx, stream, desc, T_max, n_rows, row_tok, tokens, vocab, table, hidden):
    _call("kvb_embed", ctx, stream, desc, T_max, n_rows, row_tok, tokens, vocab, table, hidden)


def kvb_qkv_proj(ctx, stream, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v,
                 ws=None, ws_bytes=0, flags=0):
    _call("kvb_qkv_proj", ctx, stream, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv,
          tok_pos, q, k, v, ws, ws_bytes, flags)


def kvb_qkv_fused(ctx, stream, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v, k_pool, v_pool,
                  n_pages, src_slot, dst_slot, alpha_mode, alpha, d_out, cksim_out, ws=None, ws_bytes=0, flags=0):
    _call("kvb_qkv_fused", ctx, stream, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v,
          k_pool, v_pool, n_pages, src_slot, dst_slot, alpha_mode, alpha, d_out, cksim_out, ws, ws_bytes, flags)


def kvb_rope(ctx, stream, desc, T_max, n_rows, row_tok, tok_pos, q, k):
    _call("kvb_rope", ctx, stream, desc, T_max, n_rows, row_tok, tok_pos, q, k)


def kvb_blend_scatter(ctx, stream, desc, T_max, n_rows, row_tok, k_rec, v_rec, k_pool, v_pool, n_pages,
                      src_slot, dst_slot, alpha_mode, alpha, d_out, cksim_out):
    _call("kvb_blend_scatter", ctx, stream, desc, T_max, n_rows, row_tok, k_rec, v_rec, k_pool,
          v_pool, n_pages, src_slot, dst_slot, alpha_mode, alpha, d_out, cksim_out)


def kvb_sparse_query_attn(ctx, stream, desc, T_max, n_rows, row_tok, tok_lo, q, k_pool, v_pool, n_pages,
                          slot_map, scale, o, ws, ws_bytes):
    _call("kvb_sparse_query_attn", ctx, stream, desc, T_max, n_rows, row_tok, tok_lo, q, k_pool,
          v_pool, n_pages, slot_map, float(scale), o, ws, ws_bytes)


def kvb_mlp(ctx, stream, desc, T_max, n_rows, row_tok, attn_o, w_o, hidden, norm2_w, w_gate_up, w_down, ws,
            ws_bytes):
    _call("kvb_mlp", ctx, stream, desc, T_max, n_rows, row_tok, attn_o, w_o, hidden, norm2_w,
          w_gate_up, w_down, ws, ws_bytes)


def kvb_deviation_topk(ctx, stream, desc, B, n_tok, cu_tok, k_rec, k_pool, n_pages, reuse_slot, k_cap, d, alpha,
                       ranking, s_count, sel, cu_rows, cursor, ws, ws_bytes):
    _call("kvb_deviation_topk", ctx, stream, desc, B, n_tok, cu_tok, k_rec, k_pool, n_pages,
          reuse_slot, k_cap, d, alpha, ranking, s_count, sel, cu_rows, cursor, ws, ws_bytes)


def kvb_deviation_topk_noalloc(ctx, stream, desc, B, n_tok, cu_tok, k_rec, k_pool, n_pages, reuse_slot, k_cap, d,
                               alpha, ranking, s_count, sel, cu_rows, cursor):
    _call("kvb_deviation_topk_noalloc", ctx, stream, desc, B, n_tok, cu_tok, k_rec, k_pool, n_pages,
          reuse_slot, k_cap, d, alpha, ranking, s_count, sel, cu_rows, cursor)


def kvb_topk(ctx, stream, desc, B, n_tok, cu_tok, d, k_cap, ranking, s_count, sel, cu_rows, cursor, ws, ws_bytes):
    _call("kvb_topk", ctx, stream, desc, B, n_tok, cu_tok, d, k_cap, ranking, s_count, sel, cu_rows, cursor, ws,
          ws_bytes)


def kvb_attnmap_deviation(ctx, stream, desc, n_tok, tok_lo, q, k_rec, k_pool, n_pages, reuse_slot, scale, dev, ws,
                          ws_bytes):
    _call("kvb_attnmap_deviation", ctx, stream, desc, n_tok, tok_lo, q, k_rec, k_pool, n_pages, reuse_slot,
          float(scale), dev, ws, ws_bytes)


def kvb_cosine_refresh(ctx, stream, desc, B, n_tok, cu_tok, T_max, cu_rows_in, sel_in, cksim, tau, rule, ranking,
                       s_count, cursor, sel_out, cu_rows_out, ws, ws_bytes):
    _call("kvb_cosine_refresh", ctx, stream, desc, B, n_tok, cu_tok, T_max, cu_rows_in, sel_in,
          cksim, float(tau), rule, ranking, s_count, cursor, sel_out, cu_rows_out, ws, ws_bytes)


def kvb_slot_map(ctx, stream, desc, B, n_tok, T_max, cu_rows, row_tok, reuse_slot, new_pages, cu_pages, slot_map,
                 dst_slot, n_pages=0, page_dirty=None):
    _call("kvb_slot_map", ctx, stream, desc, B, n_tok, T_max, cu_rows, row_tok, reuse_slot,
          new_pages, cu_pages, slot_map, dst_slot, n_pages, page_dirty)


def kvb_page_dirty_add(ctx, stream, desc, T_max, n_rows, slots, n_pages, page_dirty):
    _call("kvb_page_dirty_add", ctx, stream, desc, T_max, n_rows, slots, n_pages, page_dirty)


def kvb_link_run(ctx, stream, desc, link) -> int:
    """Queue a whole link step described by `link` (a kvb_link_desc); returns
    which selection buffer holds the set after the last layer."""
    out = c_int32(0)
    _call("kvb_link_run", ctx, stream, desc, link, ctypes.addressof(out))
    return int(out.value)
