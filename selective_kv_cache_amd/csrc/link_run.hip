// The whole link step as one call (kvb_link_run): the layer loop of
// CacheSlide's Algorithm 2 (CacheSlide page, "Method details" and
// Algorithm 2), of EPIC's LegoLink (EPIC page, section 4) or of the
// CacheBlend baseline as the EPIC page describes it (section 3.2), queued
// from the host with the per-step entry points and no host synchronisation.
//
// CacheSlide: embed every token; layer 1 recomputes all of them at their
// spliced positions into the layer's new pages; the deviation and top-k pick
// S_k; layers 2..L recompute the rows of the current selection (fusion with
// the cached K/V, alpha in the configured mode), and after each layer l with
// l % period == 0 and l < L the cosine refresh writes the next selection into
// the other buffer.  The refresh needs only the cosine similarities that the
// layer's fusion writes, so it is queued right after the fusion.  LegoLink:
// embed the static rows, recompute them in every layer (alpha = 1).
// CacheBlend: layer 1 as CacheSlide's, then the attention-map deviation and
// its top-k; layers 2..L recompute the selection, replacing the cached K/V.
//
// Launch bounds: a selective layer is launched for link->rows rows; the
// device count of the current selection (cu_rows[cur][B]) bounds the work.
#include "common.h"

namespace kvb {

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

namespace {

kvb_status check_link(kvb_ctx* ctx, const kvb_model_desc* desc, const kvb_link_desc* k) {
  KVB_CHECK_PTR(k, "link");
  if (k->mode != KVB_LINK_CACHESLIDE && k->mode != KVB_LINK_STATIC && k->mode != KVB_LINK_CACHEBLEND)
    return fail(KVB_ERR_INVALID_ARG, "bad link mode");
  if (k->B < 1 || k->n_tok < 1 || k->n_layers < 1 || k->n_pages < 1 || k->vocab < 1)
    return fail(KVB_ERR_INVALID_ARG, "B, n_tok, n_layers, n_pages and vocab must be >= 1");
  if (k->rows < 0 || k->rows > k->n_tok) return fail(KVB_ERR_INVALID_ARG, "rows outside [0, n_tok]");
  if ((long)k->n_pages * 16 > 0x7fffffffL) return fail(KVB_ERR_INVALID_ARG, "too many pages for int32 slots");
  KVB_CHECK_PTR(k->layers, "layers");
  for (int l = 0; l < k->n_layers; l++) {
    const kvb_layer_weights& w = k->layers[l];
    if (!w.norm1 || !w.w_qkv || !w.w_o || !w.norm2 || !w.w_gate_up || !w.w_down)
      return fail(KVB_ERR_INVALID_ARG, "layer " + std::to_string(l + 1) + ": a weight pointer is NULL");
  }
  KVB_CHECK_PTR(k->new_pages, "new_pages");
  KVB_CHECK_PTR(k->cu_pages, "cu_pages");
  for (int l = 0; l < k->n_layers; l++)
    if (!k->new_pages[l] || !k->cu_pages[l])
      return fail(KVB_ERR_INVALID_ARG, "layer " + std::to_string(l + 1) + ": new_pages or cu_pages is NULL");
  KVB_CHECK_PTR(k->embedding, "embedding");
  KVB_CHECK_PTR(k->tokens, "tokens");
  KVB_CHECK_PTR(k->pos, "pos");
  KVB_CHECK_PTR(k->lo, "lo");
  KVB_CHECK_PTR(k->cu_tok, "cu_tok");
  KVB_CHECK_PTR(k->reuse_slot, "reuse_slot");
  KVB_CHECK_PTR(k->page_table, "page_table");
  KVB_CHECK_PTR(k->k_pool, "k_pool");
  KVB_CHECK_PTR(k->v_pool, "v_pool");
  KVB_CHECK_PTR(k->hidden, "hidden");
  KVB_CHECK_PTR(k->q, "q");
  KVB_CHECK_PTR(k->k, "k");
  KVB_CHECK_PTR(k->v, "v");
  KVB_CHECK_PTR(k->o, "o");
  KVB_CHECK_PTR(k->dst_slot, "dst_slot");
  if (k->mode == KVB_LINK_CACHESLIDE) {
    if (k->period < 1) return fail(KVB_ERR_INVALID_ARG, "period < 1");
    if (k->refresh_rule != KVB_REFRESH_LITERAL && k->refresh_rule != KVB_REFRESH_DISSIM)
      return fail(KVB_ERR_INVALID_ARG, "bad refresh_rule");
    if (k->alpha_mode != KVB_ALPHA_LAG && k->alpha_mode != KVB_ALPHA_CURRENT && k->alpha_mode != KVB_ALPHA_ONE)
      return fail(KVB_ERR_INVALID_ARG, "bad alpha_mode");
    KVB_CHECK_PTR(k->k_cap, "k_cap");
    KVB_CHECK_PTR(k->d, "d");
    KVB_CHECK_PTR(k->alpha, "alpha");
    KVB_CHECK_PTR(k->dev, "dev");
    KVB_CHECK_PTR(k->cksim, "cksim");
    KVB_CHECK_PTR(k->ranking, "ranking");
    KVB_CHECK_PTR(k->s_count, "s_count");
    KVB_CHECK_PTR(k->cursor, "cursor");
    KVB_CHECK_PTR(k->sel[0], "sel[0]");
    KVB_CHECK_PTR(k->sel[1], "sel[1]");
    KVB_CHECK_PTR(k->cu_rows[0], "cu_rows[0]");
    KVB_CHECK_PTR(k->cu_rows[1], "cu_rows[1]");
    if (k->sel[0] == k->sel[1] || k->cu_rows[0] == k->cu_rows[1])
      return fail(KVB_ERR_INVALID_ARG, "the two selection buffers must differ");
  } else if (k->mode == KVB_LINK_CACHEBLEND) {
    KVB_CHECK_PTR(k->k_cap, "k_cap");
    KVB_CHECK_PTR(k->d, "d");
    KVB_CHECK_PTR(k->ranking, "ranking");
    KVB_CHECK_PTR(k->s_count, "s_count");
    KVB_CHECK_PTR(k->cursor, "cursor");
    KVB_CHECK_PTR(k->sel[0], "sel[0]");
    KVB_CHECK_PTR(k->cu_rows[0], "cu_rows[0]");
  } else if (k->rows > 0) {
    KVB_CHECK_PTR(k->static_rows, "static_rows");
    KVB_CHECK_PTR(k->static_cu, "static_cu");
  }
  size_t need = 0;
  KVB_TRY(kvb_workspace_size(ctx, desc, k->n_tok, k->n_tok, k->B, &need));
  if (!k->ws || k->ws_bytes < need) return fail(KVB_ERR_WORKSPACE, "kvb_link_run workspace too small");
  return KVB_OK;
}

// One recomputed layer (1-based l) over T rows: slot map, Q/K/V + RoPE +
// fusion and scatter (then `after_blend`), attention, O-projection + MLP.
template <class F>
kvb_status layer_rows(kvb_ctx* ctx, void* st, const kvb_model_desc* desc, const kvb_link_desc* k, int l, int T,
                      const int32_t* n_rows, const int32_t* rows, const int32_t* cu_rows, const int32_t* src_slot,
                      int32_t alpha_mode, float* alpha, float* d_out, float* cksim_out, F after_blend) {
  const size_t N = (size_t)k->n_tok;
  const kvb_layer_weights& w = k->layers[l - 1];
  int32_t* slot_map = k->page_table + (size_t)(l - 1) * N;
  KVB_TRY(kvb_slot_map(ctx, st, desc, k->B, k->n_tok, T, cu_rows, rows, k->reuse_slot + (size_t)(l - 1) * N,
                       k->new_pages[l - 1], k->cu_pages[l - 1], slot_map, k->dst_slot, k->n_pages,
                       l >= 2 ? k->page_dirty : nullptr));
  // layer 1 batch-invariant (its keys must equal the compile step's bit for
  // bit where nothing moved); the selective layers may split K
  const int32_t flags = l == 1 ? KVB_QKV_BATCH_INVARIANT : KVB_QKV_SPLIT_K;
  KVB_TRY(kvb_qkv_fused(ctx, st, desc, T, n_rows, rows, k->hidden, w.norm1, w.w_qkv, k->pos, k->q, k->k, k->v,
                        k->k_pool, k->v_pool, k->n_pages, src_slot, k->dst_slot, alpha_mode, alpha, d_out,
                        cksim_out, k->ws, k->ws_bytes, flags));
  KVB_TRY(after_blend());
  KVB_TRY(kvb_sparse_query_attn(ctx, st, desc, T, n_rows, rows, k->lo, k->q, k->k_pool, k->v_pool, k->n_pages,
                                slot_map, k->scale, k->o, k->ws, k->ws_bytes));
  return kvb_mlp(ctx, st, desc, T, n_rows, rows, k->o, w.w_o, k->hidden, w.norm2, w.w_gate_up, w.w_down, k->ws,
                 k->ws_bytes);
}

// page tables of layers whose rows were all skipped: the reused slots
kvb_status reuse_tables(kvb_ctx* ctx, void* st, const kvb_model_desc* desc, const kvb_link_desc* k, int l0) {
  const size_t N = (size_t)k->n_tok;
  for (int l = l0; l <= k->n_layers; l++)
    KVB_TRY(kvb_slot_map(ctx, st, desc, k->B, k->n_tok, 0, nullptr, nullptr, k->reuse_slot + (size_t)(l - 1) * N,
                         nullptr, nullptr, k->page_table + (size_t)(l - 1) * N, nullptr, k->n_pages, nullptr));
  return KVB_OK;
}

}  // namespace
}  // namespace kvb

using namespace kvb;

extern "C" kvb_status kvb_link_run(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, const kvb_link_desc* k,
                                   int32_t* final_sel) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  KVB_TRY(check_link(ctx, desc, k));
  auto nothing = [] { return KVB_OK; };
  int cur = 0;
  {
    CtxScope scope(ctx);
    if (k->page_dirty) {
      hipStream_t st = (hipStream_t)stream;
      fill_i32_kernel<<<cdiv(k->n_pages, 256), 256, 0, st>>>(k->page_dirty, k->n_pages, 0);
      KVB_TRY(check_launch("fill_i32_kernel"));
    }
  }
  if (k->mode == KVB_LINK_STATIC) {
    const int T = k->rows;
    if (T == 0) {
      KVB_TRY(reuse_tables(ctx, stream, desc, k, 1));
    } else {
      KVB_TRY(kvb_embed(ctx, stream, desc, T, nullptr, k->static_rows, k->tokens, k->vocab, k->embedding, k->hidden));
      for (int l = 1; l <= k->n_layers; l++)
        KVB_TRY(layer_rows(ctx, stream, desc, k, l, T, nullptr, k->static_rows, k->static_cu, nullptr, KVB_ALPHA_ONE,
                           nullptr, nullptr, nullptr, nothing));
    }
  } else if (k->mode == KVB_LINK_CACHEBLEND) {
    const int N = k->n_tok, B = k->B, T = k->rows;
    KVB_TRY(kvb_embed(ctx, stream, desc, N, nullptr, nullptr, k->tokens, k->vocab, k->embedding, k->hidden));
    KVB_TRY(layer_rows(ctx, stream, desc, k, 1, N, nullptr, nullptr, k->cu_tok, nullptr, KVB_ALPHA_ONE, nullptr,
                       nullptr, nullptr, nothing));
    // q and k still hold layer 1's queries and recomputed keys of every token
    KVB_TRY(kvb_attnmap_deviation(ctx, stream, desc, N, k->lo, k->q, k->k, k->k_pool, k->n_pages, k->reuse_slot,
                                  k->scale, k->d, k->ws, k->ws_bytes));
    KVB_TRY(kvb_topk(ctx, stream, desc, B, N, k->cu_tok, k->d, k->k_cap, k->ranking, k->s_count, k->sel[0],
                     k->cu_rows[0], k->cursor, k->ws, k->ws_bytes));
    if (T == 0) {
      KVB_TRY(reuse_tables(ctx, stream, desc, k, 2));
    } else {
      for (int l = 2; l <= k->n_layers; l++)
        KVB_TRY(layer_rows(ctx, stream, desc, k, l, T, k->cu_rows[0] + B, k->sel[0], k->cu_rows[0], nullptr,
                           KVB_ALPHA_ONE, nullptr, nullptr, nullptr, nothing));
    }
  } else {
    const int N = k->n_tok, B = k->B, T = k->rows;
    KVB_TRY(kvb_embed(ctx, stream, desc, N, nullptr, nullptr, k->tokens, k->vocab, k->embedding, k->hidden));
    // layer 1: every token at its spliced position, into layer 1's new pages
    KVB_TRY(layer_rows(ctx, stream, desc, k, 1, N, nullptr, nullptr, k->cu_tok, nullptr, KVB_ALPHA_ONE, nullptr,
                       nullptr, nullptr, nothing));
    KVB_TRY(kvb_deviation_topk(ctx, stream, desc, B, N, k->cu_tok, k->k, k->k_pool, k->n_pages, k->reuse_slot,
                               k->k_cap, k->d, k->alpha, k->ranking, k->s_count, k->sel[0], k->cu_rows[0], k->cursor,
                               k->ws, k->ws_bytes));
    if (T == 0) {
      KVB_TRY(reuse_tables(ctx, stream, desc, k, 2));
    } else {
      for (int l = 2; l <= k->n_layers; l++) {
        const bool refresh = l % k->period == 0 && l < k->n_layers;
        const int c = cur;
        auto refresh_now = [&]() {
          return kvb_cosine_refresh(ctx, stream, desc, B, N, k->cu_tok, T, k->cu_rows[c], k->sel[c], k->cksim, k->tau,
                                    k->refresh_rule, k->ranking, k->s_count, k->cursor, k->sel[1 - c],
                                    k->cu_rows[1 - c], k->ws, k->ws_bytes);
        };
        const int32_t* n_rows = k->cu_rows[c] + B;  // the selection's device row count
        if (refresh)
          KVB_TRY(layer_rows(ctx, stream, desc, k, l, T, n_rows, k->sel[c], k->cu_rows[c],
                             k->reuse_slot + (size_t)(l - 1) * N, k->alpha_mode, k->alpha, k->dev, k->cksim,
                             refresh_now));
        else
          KVB_TRY(layer_rows(ctx, stream, desc, k, l, T, n_rows, k->sel[c], k->cu_rows[c],
                             k->reuse_slot + (size_t)(l - 1) * N, k->alpha_mode, k->alpha, k->dev, nullptr, nothing));
        if (refresh) cur = 1 - cur;
      }
    }
  }
  if (final_sel) *final_sel = cur;
  return KVB_OK;
}
