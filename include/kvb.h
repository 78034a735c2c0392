/*
 * kvb.h - C ABI of the link-step library for selective KV recompute over a
 * spliced, position-shifted reused KV cache, built for AMD Instinct MI355X
 * (gfx950).
 *
 * The method: the KV caches of several chunks, each compiled alone from
 * position 0 (EPIC page, section 3.1, compile step), are spliced into one
 * request and a subset of tokens is recomputed (link step).  Three ways of
 * choosing the subset are served by the same calls:
 *   - CacheSlide Weighted Correction Attention (CacheSlide page, "Method
 *     details", weighted-correction paragraphs and Algorithm 2): layer 1
 *     recomputes every token and ranks them by d_i = ||K_i^rec - K_i^reuse||^2;
 *     layers 2..L recompute the top-k and fuse
 *     K_i <- alpha_i K_i^rec + (1 - alpha_i) K_i^reuse (same for V) with
 *     alpha_i = d_i / ||K_i^reuse||^2; every four layers a cosine check
 *     retires tokens and refills from the ranking;
 *   - EPIC LegoLink (EPIC page, section 4): the first k tokens of every chunk
 *     but the first, plus the user's uncached query tokens, recomputed in
 *     every layer, replacing the cached K/V;
 *   - the CacheBlend baseline as the EPIC page describes it (section 3.2):
 *     layer 1 recomputes every token, the tokens whose attention maps under
 *     the cached and the recomputed keys differ most are recomputed in layers
 *     2..L, replacing the cached K/V (kvb_attnmap_deviation, kvb_topk).
 * Recomputed K/V go to freshly allocated pages (CacheSlide page, SLIDE
 * implementation paragraph) of a paged cache with 16-token pages.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All calls are enqueue-only on the given HIP stream (a hipStream_t passed
 *    as void*; NULL = the default stream) and never synchronise the device.
 *  - Arguments are validated on the host before anything is enqueued; on error
 *    nothing is enqueued, a status < 0 is returned and kvb_last_error() gives a
 *    thread-local message.  A failed kernel launch returns KVB_ERR_HIP.
 *  - Every device buffer is allocated and owned by the caller; the library
 *    allocates no device memory in these calls and keeps no pointer after a
 *    call returns.  Buffers are row-major, contiguous and 16-byte aligned.
 *  - Storage type (desc->dtype): KVB_F32 (float) or KVB_BF16 (bfloat16 bits
 *    in uint16).  Weights, embeddings, hidden state, Q/K/V, attention output
 *    and the KV pool all use it; reductions and softmax run in float32.
 *  - Token space: the requests of a batch are concatenated; token g of the
 *    batch is "global token g", 0 <= g < n_tok.  Per-token int32 arrays
 *    indexed by g: tok_pos[g] = RoPE position, tok_lo[g] = first key index
 *    visible to g (the start of its request, or of its chunk at compile time).
 *  - Row batches: a call works on T rows; row r is global token row_tok[r]
 *    (row_tok == NULL means row r is token r).  T_max is a host bound used
 *    for launch sizes; n_rows (device int32, may be NULL = T_max) holds the
 *    actual count, so counts produced on the device need no host round trip.
 *    Rows >= *n_rows are neither read nor written.
 *  - KV pool: K and V are separate arrays of n_pages pages, each
 *    [n_kv_heads][page_size][head_dim]; slot s lives in page s / page_size at
 *    position s % page_size.  Slots outside [0, n_pages*page_size) are skipped
 *    by the kernels (never dereferenced).
 */
#ifndef KVB_H
#define KVB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvb_status;
#define KVB_OK 0
#define KVB_ERR_INVALID_ARG (-1)  /* null pointer, negative size, inconsistent shape */
#define KVB_ERR_UNSUPPORTED (-2)  /* dtype, head_dim not in {64,128}, page_size != 16, bf16 dims not multiples of 64 */
#define KVB_ERR_HIP (-3)          /* HIP runtime / launch error */
#define KVB_ERR_CAPACITY (-4)     /* page pool exhausted */
#define KVB_ERR_WORKSPACE (-5)    /* workspace missing or too small */

#define KVB_F32 0
#define KVB_BF16 1

/* alpha handling of kvb_blend_scatter */
#define KVB_ALPHA_LAG 0      /* blend with the stored alpha, then store this layer's alpha (Algorithm 2 order) */
#define KVB_ALPHA_CURRENT 1  /* blend with this layer's alpha and store it */
#define KVB_ALPHA_ONE 2      /* alpha = 1: the recomputed rows replace the cached ones; nothing stored */

/* retire rule of kvb_cosine_refresh */
#define KVB_REFRESH_LITERAL 0  /* retire when CKSim < tau (the pages' stated test) */
#define KVB_REFRESH_DISSIM 1   /* retire when CKSim > 1 - tau (alternative reading) */

typedef struct kvb_model_desc {
  int32_t d_model;     /* hidden size d */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv, divides Hq */
  int32_t head_dim;    /* 64 or 128 */
  int32_t ffn;         /* SwiGLU inner size F */
  int32_t page_size;   /* must be 16 */
  float rope_base;     /* RoPE base, e.g. 10000 */
  float rms_eps;       /* RMSNorm epsilon */
  int32_t dtype;       /* KVB_F32 or KVB_BF16 */
} kvb_model_desc;

typedef struct kvb_ctx kvb_ctx;
typedef struct kvb_pool kvb_pool;

/* ----------------------------------------------------------------- basics */

const char* kvb_status_string(kvb_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* kvb_last_error(void);

/* Context bound to HIP device `device` (queried once for its CU count).
 * A context is used by one host thread at a time. */
kvb_status kvb_create(int32_t device, kvb_ctx** out);
kvb_status kvb_destroy(kvb_ctx* ctx);

/* Bytes of workspace the calls below need for batches of at most max_rows
 * rows, max_tokens tokens and max_requests requests. */
kvb_status kvb_workspace_size(kvb_ctx* ctx, const kvb_model_desc* desc, int32_t max_rows,
                              int32_t max_tokens, int32_t max_requests, size_t* bytes);

/* Launch timing (tracing).  With filter != NULL, every later kernel launch of
 * this context whose kernel name contains `filter` ("" = all) is bracketed with
 * HIP events on its stream; filter == NULL turns timing off.  Kernel names:
 * embed, rmsnorm, gemm_qkv, rope, blend_scatter, attention, attention_merge, gemm_oproj, gemm_swiglu,
 * gemm_down, splitk_reduce, deviation, topk_sort, topk_rank, topk_compact, refresh_flag,
 * refresh_compact, slot_copy, slot_scatter, page_dirty, rope_fuse, attnmap, attnmap_reduce. */
kvb_status kvb_timing_enable(kvb_ctx* ctx, const char* filter);
/* Waits for the recorded events and folds them into per-kernel totals, then
 * sets *needed to the size of the JSON text {"name": {"count": n, "ms": t}, ...}
 * (first-seen order, NUL included).  If buf holds at least that many bytes the
 * text is copied and the totals are cleared; otherwise they are kept (call
 * again with a large enough buffer). */
kvb_status kvb_timing_read(kvb_ctx* ctx, char* buf, size_t len, size_t* needed);

/* --------------------------------------------------- host page allocator
 * Deterministic allocator over page ids 0..n_pages-1: kvb_pool_alloc hands out
 * the n lowest free ids in ascending order, or fails with KVB_ERR_CAPACITY
 * and allocates nothing (SLIDE preallocation of new pages, CacheSlide page,
 * SLIDE implementation paragraph).  Host memory only. */
kvb_status kvb_pool_create(int32_t n_pages, kvb_pool** out);
kvb_status kvb_pool_destroy(kvb_pool* pool);
kvb_status kvb_pool_alloc(kvb_pool* pool, int32_t n, int32_t* out_ids /* host [n] */);
kvb_status kvb_pool_release(kvb_pool* pool, int32_t n, const int32_t* ids /* host [n] */);
kvb_status kvb_pool_free_count(const kvb_pool* pool, int32_t* out);

/* --------------------------------------------------- page tiers
 * Copy whole pages between a host tier and the device pool (CacheSlide page,
 * SLIDE: reused KV that lives in a lower tier is loaded layer by layer while
 * the selected rows are recomputed into new pages).  Both sides use the pool
 * layout [page][Hkv][16][hd] with page p at byte offset p * page_bytes, so a
 * host mirror of the first P pages serves pages 0..P-1.  page_ids: host int32
 * [n_ids], non-negative; runs of consecutive ids become one hipMemcpyAsync
 * each (K, then V) on `stream`, so the call returns once they are enqueued.
 * dst_k or dst_v may be NULL to copy one half only (layer 1 of CacheSlide
 * reads reused keys only).  direction: KVB_COPY_H2D (src host, dst device) or
 * KVB_COPY_D2H.  Host buffers must be pinned for the copies to overlap
 * kernels.  The caller keeps ids within both buffers; the library cannot
 * check host extents. */
#define KVB_COPY_H2D 0
#define KVB_COPY_D2H 1
kvb_status kvb_pages_copy(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t direction,
                          const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                          const int32_t* page_ids /* host [n_ids] */, int32_t n_ids);

/* ------------------------------------------------------------ the path */

/* hidden[row_tok[r]] = table[tokens[row_tok[r]]] for r < *n_rows.
 * First step of every recomputed token at layer 1 (EPIC page, section 4,
 * LegoLink step 1: embeddings E of the selected tokens).  tokens: device int32
 * [n_tok] vocabulary ids in [0, vocab) (rows with other ids are skipped);
 * table: [vocab, d]; hidden: [n_tok, d]. */
kvb_status kvb_embed(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                     const int32_t* n_rows, const int32_t* row_tok, const int32_t* tokens,
                     int32_t vocab, const void* table, void* hidden);

/* Gathered-row RMSNorm + Q/K/V projection (EPIC page, section 4, LegoLink
 * step 2: Q, K, V = E W for the recomputed rows only).
 *   a_r = RMSNorm(hidden[row_tok[r]]) * norm_w;  [q|k|v]_r = a_r W_qkv^T
 * hidden [n_tok, d]; norm_w [d]; w_qkv [(Hq + 2 Hkv) * hd, d] (Q rows, then K,
 * then V); outputs q [T, Hq, hd], k [T, Hkv, hd], v [T, Hkv, hd].
 * If tok_pos != NULL, rotate-half RoPE at position tok_pos[row_tok[r]] is
 * applied to q and k (as kvb_rope).
 * flags = KVB_QKV_BATCH_INVARIANT (0): the per-row result does not depend on
 * T, on the row's place in the batch or on the other rows (a chunk seen at
 * the same positions in compile and link gets bitwise-equal keys); use it for
 * the compile step and for layer 1 of a link step.  flags = KVB_QKV_SPLIT_K:
 * for bf16 the K reduction may also be split across blocks (partials added in
 * a fixed order, so results stay deterministic but depend on T); for rows
 * whose keys are never compared bitwise with another call's (decode tokens,
 * the selective layers), where a few rows would otherwise leave most of the
 * GPU idle.
 * norm_w == NULL means unit gains.  With bf16 storage a_r is written to the
 * workspace rounded to bf16 once (ws_bytes >= kvb_workspace_size for T_max
 * rows); float32 storage needs no workspace (ws may be NULL). */
#define KVB_QKV_BATCH_INVARIANT 0
#define KVB_QKV_SPLIT_K 1
kvb_status kvb_qkv_proj(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                        const int32_t* n_rows, const int32_t* row_tok, const void* hidden,
                        const void* norm_w, const void* w_qkv, const int32_t* tok_pos, void* q,
                        void* k, void* v, void* ws, size_t ws_bytes, int32_t flags);

/* Q/K/V projection, RoPE, and the fusion + scatter of the recomputed K/V
 * into the page pool: what kvb_qkv_proj (with tok_pos) followed by
 * kvb_blend_scatter on its k and v computes (EPIC page, section 4, LegoLink
 * step 2; CacheSlide page, Algorithm 2 fusion line and alpha definition;
 * SLIDE's new pages), with the rotation, the fusion and the scatter done in
 * one pass over each row after the projection.  The arguments are
 * kvb_qkv_proj's, then kvb_blend_scatter's from k_pool on (dst_slot required;
 * src_slot NULL: KVB_ALPHA_ONE only and d_out / cksim_out NULL), then ws,
 * ws_bytes and flags as for kvb_qkv_proj.  q, k, v and every pool, alpha,
 * d_out and cksim_out value are those of the two-call sequence.  Workspace:
 * kvb_workspace_size. */
kvb_status kvb_qkv_fused(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                         const int32_t* n_rows, const int32_t* row_tok, const void* hidden,
                         const void* norm_w, const void* w_qkv, const int32_t* tok_pos, void* q,
                         void* k, void* v, void* k_pool, void* v_pool, int32_t n_pages,
                         const int32_t* src_slot, const int32_t* dst_slot, int32_t alpha_mode,
                         float* alpha, float* d_out, float* cksim_out, void* ws, size_t ws_bytes,
                         int32_t flags);

/* In-place rotate-half RoPE of q [T, Hq, hd] and k [T, Hkv, hd] at positions
 * tok_pos[row_tok[r]]: pair (j, j + hd/2) rotated by pos * base^(-2j/hd).
 * Recomputed tokens are given their correct absolute positions in the
 * spliced prompt, while the compile step encodes every chunk from position 0
 * (EPIC page, section 4.1), so the link step passes global positions and the
 * compile step chunk-local ones.  Angles are formed in double precision. */
kvb_status kvb_rope(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                    const int32_t* n_rows, const int32_t* row_tok, const int32_t* tok_pos, void* q,
                    void* k);

/* Fusion and scatter of the recomputed rows into the page pool (CacheSlide
 * page, Algorithm 2 fusion line and alpha definition; SLIDE writes the
 * selected tokens' K/V into newly allocated pages).  For each row r < *n_rows
 * with token g = row_tok[r]:
 *   reuse = pool rows at src_slot[g] (the token's cached K/V of this layer)
 *   d_r   = ||k_rec_r - k_reuse||^2 (whole row, all KV heads), float32
 *   a_new = d_r / ||k_reuse||^2   (0 if both are 0, 1 if only the norm is 0)
 *   a_use = alpha[g] (KVB_ALPHA_LAG), a_new (KVB_ALPHA_CURRENT) or 1 (KVB_ALPHA_ONE)
 *   K, V at dst_slot[r] <- a_use * rec + (1 - a_use) * reuse  (float32, one rounding)
 *   alpha[g] <- a_new unless KVB_ALPHA_ONE;  d_out[r] <- d_r;
 *   cksim_out[r] <- mean over KV heads of cos(k_rec_r,h, k_reuse_h)
 *                   (1 if both vectors are 0, 0 if exactly one is).
 * src_slot == NULL means "no cached row": only KVB_ALPHA_ONE is allowed and
 * d_out / cksim_out must be NULL (compile step, layer 1, LegoLink).
 * k_rec, v_rec [T, Hkv, hd]; alpha [n_tok] float; d_out, cksim_out [T] float
 * or NULL; dst_slot [T]; src_slot [n_tok]. */
kvb_status kvb_blend_scatter(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                             const int32_t* n_rows, const int32_t* row_tok, const void* k_rec,
                             const void* v_rec, void* k_pool, void* v_pool, int32_t n_pages,
                             const int32_t* src_slot, const int32_t* dst_slot, int32_t alpha_mode,
                             float* alpha, float* d_out, float* cksim_out);

/* Causal grouped-query attention of gathered query rows over the full spliced
 * KV of the layer (EPIC page, section 4, LegoLink steps 3-5:
 * A = softmax(Q K_exp^T, causal) over all N tokens, O = A V_exp).  Row r
 * (token g = row_tok[r]) attends the keys j with tok_lo[g] <= j <= g, read
 * from slot slot_map[j] of the pools; query head h reads KV head
 * h / (Hq / Hkv); scores are scaled by `scale`.  A key whose slot lies
 * outside [0, 16 n_pages) is left out of the softmax, as if masked; a row
 * with no key left gets O = 0.
 * q [T, Hq, hd]; slot_map [n_tok]; o [T, Hq * hd].  bf16 splits long key
 * ranges over several workgroups when ws holds the partial results
 * (kvb_workspace_size); with less workspace it runs unsplit. */
kvb_status kvb_sparse_query_attn(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc,
                                 int32_t T_max, const int32_t* n_rows, const int32_t* row_tok,
                                 const int32_t* tok_lo, const void* q, const void* k_pool,
                                 const void* v_pool, int32_t n_pages, const int32_t* slot_map,
                                 float scale, void* o, void* ws, size_t ws_bytes);

/* Output projection and SwiGLU MLP of the recomputed rows (EPIC page,
 * section 4, LegoLink step 5: O = A V_exp W_O, the layer output):
 *   h1 = hidden[g] + o_r W_o^T ;  b = RMSNorm(h1) * norm2_w ;
 *   hidden[g] <- h1 + (silu(b W_gate^T) * (b W_up^T)) W_down^T
 * o [T, Hq*hd]; w_o [d, Hq*hd]; w_gate_up [2F, d] (gate rows then up rows);
 * w_down [d, F]; hidden [n_tok, d] updated in place at rows row_tok[r].
 * Needs workspace (kvb_workspace_size). */
kvb_status kvb_mlp(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                   const int32_t* n_rows, const int32_t* row_tok, const void* attn_o,
                   const void* w_o, void* hidden, const void* norm2_w, const void* w_gate_up,
                   const void* w_down, void* ws, size_t ws_bytes);

/* Layer-1 deviation and top-k selection of CacheSlide (CacheSlide page,
 * Algorithm 2 initialisation: d_i, alpha_i for every token, S = {d_i > 0},
 * S_k = top-k of S by d).  For request b (tokens cu_tok[b] .. cu_tok[b+1]-1):
 *   d[g]     = ||k_rec[g] - k_reuse(g)||^2, reuse read at slot reuse_slot[g]
 *   alpha[g] = d[g] / ||k_reuse(g)||^2   (zero-norm rule as kvb_blend_scatter)
 *   ranking[cu_tok[b] + i] = the i-th token of S by d descending, ties by
 *     lower index; entries from s_count[b] on list the d == 0 tokens ascending
 *   s_count[b] = |S|;  k_b = min(k_cap[b], |S|);  cursor[b] = k_b
 *   sel[cu_rows[b] .. cu_rows[b+1]-1] = the k_b top tokens in ascending order
 *   cu_rows[0] = 0, cu_rows[b+1] = cu_rows[b] + k_b
 * k_rec is token-indexed [n_tok, Hkv, hd] (layer 1 recomputes every token);
 * cu_tok, k_cap device int32; d, alpha float [n_tok]; ranking, sel int32
 * [n_tok]; s_count, cursor int32 [B]; cu_rows int32 [B+1].  Needs workspace.
 * Results are bitwise deterministic. */
kvb_status kvb_deviation_topk(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B,
                              int32_t n_tok, const int32_t* cu_tok, const void* k_rec,
                              const void* k_pool, int32_t n_pages, const int32_t* reuse_slot,
                              const int32_t* k_cap, float* d, float* alpha, int32_t* ranking,
                              int32_t* s_count, int32_t* sel, int32_t* cu_rows, int32_t* cursor,
                              void* ws, size_t ws_bytes);

/* Allocation-free variant of kvb_deviation_topk, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * kvb_deviation_topk, without ws / ws_bytes: the top-k keys and flags live in
 * a fixed 2 MiB device array of the library (one per GPU, held until the
 * process ends, its address looked up in kvb_create or on the first call on a
 * device).  Batches of more than KVB_NOALLOC_MAX_TOKENS tokens or
 * KVB_NOALLOC_MAX_REQUESTS requests are refused with KVB_ERR_WORKSPACE before
 * anything is enqueued.  The call allocates nothing.  Every call on a GPU
 * shares that GPU's array: calls that may overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller. */
#define KVB_NOALLOC_MAX_TOKENS 131072
#define KVB_NOALLOC_MAX_REQUESTS 4096
kvb_status kvb_deviation_topk_noalloc(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B,
                                      int32_t n_tok, const int32_t* cu_tok, const void* k_rec,
                                      const void* k_pool, int32_t n_pages, const int32_t* reuse_slot,
                                      const int32_t* k_cap, float* d, float* alpha, int32_t* ranking,
                                      int32_t* s_count, int32_t* sel, int32_t* cu_rows, int32_t* cursor);

/* Top-k selection from a per-token score already computed (the ranking, S and
 * S_k rules of kvb_deviation_topk, for a selection whose score is not the key
 * deviation, e.g. kvb_attnmap_deviation).  d [n_tok] float (>= 0) is read
 * only; every other argument and the results are as in kvb_deviation_topk.
 * Needs workspace.  Results are bitwise deterministic. */
kvb_status kvb_topk(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B,
                    int32_t n_tok, const int32_t* cu_tok, const float* d, const int32_t* k_cap,
                    int32_t* ranking, int32_t* s_count, int32_t* sel, int32_t* cu_rows,
                    int32_t* cursor, void* ws, size_t ws_bytes);

/* Attention-map deviation of the CacheBlend-style selection (EPIC page,
 * section 3.2, the CacheBlend baseline: after layer 1 is recomputed for every
 * token, each token's attention map under the cached keys is compared with
 * its map under the recomputed keys; the tokens that differ most are
 * recomputed in the later layers).  For every token g:
 *   dev[g] = (1 / Hq) sum_h sum_{j = tok_lo[g] .. g} |Pn[h,g,j] - Po[h,g,j]|
 *   Pn[h,g,:] = softmax_j(scale * q[g,h] . k_rec[j, h / G])
 *   Po[h,g,:] = softmax_j(scale * q[g,h] . key at slot reuse_slot[j] of k_pool, head h / G)
 * with G = Hq / Hkv, i.e. the L1 distance of the two attention rows, mean over
 * query heads, in [0, 2].  q [n_tok, Hq, hd] and k_rec [n_tok, Hkv, hd] are
 * token-indexed (layer 1 recomputes every token); k_pool [n_pages, Hkv, 16,
 * hd]; tok_lo, reuse_slot device int32 [n_tok]; dev float [n_tok].  A key
 * whose reuse slot is outside the pool is left out of both maps; a token with
 * no visible key gets 0.  bf16 needs n_q_heads / n_kv_heads to be a power of
 * two up to 32 and workspace (kvb_workspace_size for max_tokens >= n_tok);
 * fp32 needs n_q_heads <= 256 and no workspace.  Results are bitwise
 * deterministic. */
kvb_status kvb_attnmap_deviation(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc,
                                 int32_t n_tok, const int32_t* tok_lo, const void* q,
                                 const void* k_rec, const void* k_pool, int32_t n_pages,
                                 const int32_t* reuse_slot, float scale, float* dev, void* ws,
                                 size_t ws_bytes);

/* Similarity-gated refresh (CacheSlide page, Algorithm 2, every four layers:
 * a token of S_k whose CKSim is below tau leaves S_k and S, and the token of
 * S \ S_k with the largest deviation joins).  Works on a snapshot: for
 * request b with rows cu_rows_in[b] .. cu_rows_in[b+1]-1 of sel_in and their
 * cksim values, R_b = rows to retire under `rule`; the next
 * m_b = min(|R_b|, s_count[b] - cursor[b]) tokens of the ranking (from
 * ranking[cu_tok[b] + cursor[b]]) join; cursor[b] += m_b.  The new set, in
 * ascending order, goes to sel_out at cu_rows_out[b] (cu_rows_out[0] = 0).
 * sel_in and sel_out must not overlap.  Needs workspace. */
kvb_status kvb_cosine_refresh(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B,
                              int32_t n_tok, const int32_t* cu_tok, int32_t T_max,
                              const int32_t* cu_rows_in, const int32_t* sel_in,
                              const float* cksim, float tau, int32_t rule,
                              const int32_t* ranking, const int32_t* s_count, int32_t* cursor,
                              int32_t* sel_out, int32_t* cu_rows_out, void* ws, size_t ws_bytes);

/* Slot map of one layer (SLIDE: selected tokens are routed to the layer's new
 * pages through the request's slot mapping).  slot_map[g] = reuse_slot[g] for
 * every token, then for each row r of request b (rank j = r - cu_rows[b]):
 *   dst_slot[r] = new_pages[cu_pages[b] + j / page_size] * page_size + j % page_size
 *   slot_map[row_tok[r]] = dst_slot[r]
 * Rows whose rank exceeds the request's page list get dst_slot = -1 and keep
 * their reuse slot.  reuse_slot may be NULL (slot_map starts at -1).
 * row_tok NULL = identity (then cu_rows doubles as cu_tok).
 * page_dirty (device int32 [n_pages], or NULL): SLIDE's per-page dirty
 * counters (CacheSlide page, SLIDE implementation paragraph: from layer 2 on,
 * a page holding selected tokens is dirty, and its counter is updated whenever
 * the slot mapping routes a selected token to it): page_dirty[dst_slot[r] /
 * page_size] += 1 for every row given a slot below n_pages * page_size.  The
 * caller clears the counters when it starts a link step and passes them for
 * the selective layers (2..L) only. */
kvb_status kvb_slot_map(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B,
                        int32_t n_tok, int32_t T_max, const int32_t* cu_rows,
                        const int32_t* row_tok, const int32_t* reuse_slot,
                        const int32_t* new_pages, const int32_t* cu_pages, int32_t* slot_map,
                        int32_t* dst_slot, int32_t n_pages, int32_t* page_dirty);

/* Dirty-page counters during decode (CacheSlide page, SLIDE: the policy of
 * the link step applies during decode as well, whose tokens are written
 * first into the superseded slots of the selected tokens, then into fresh
 * pages).  For r < *n_rows (n_rows NULL = T_max): if 0 <= slots[r] <
 * n_pages * page_size, page_dirty[slots[r] / page_size] += 1.  slots: device
 * int32 [T_max], the slots the K/V of the rows were written to;
 * page_dirty: device int32 [n_pages].  Counts are exact whatever the order of
 * the increments. */
kvb_status kvb_page_dirty_add(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                              const int32_t* n_rows, const int32_t* slots, int32_t n_pages,
                              int32_t* page_dirty);

/* ------------------------------------------------------ the whole link step */

/* Weights of one layer (device pointers, storage type desc->dtype). */
typedef struct kvb_layer_weights {
  const void* norm1;      /* [d] RMSNorm gain before Q/K/V */
  const void* w_qkv;      /* [(Hq + 2 Hkv) hd, d] */
  const void* w_o;        /* [d, Hq hd] */
  const void* norm2;      /* [d] RMSNorm gain before the MLP */
  const void* w_gate_up;  /* [2 F, d]: gate rows, then up rows */
  const void* w_down;     /* [d, F] */
} kvb_layer_weights;

#define KVB_LINK_CACHESLIDE 0  /* layer 1 in full, deviation top-k, fusion and refresh in layers 2..L */
#define KVB_LINK_STATIC 1      /* a fixed row set recomputed in every layer, replacing the cached K/V */
#define KVB_LINK_CACHEBLEND 2  /* layer 1 in full, attention-map deviation top-k, those rows replace the cached K/V */

/* Everything one link step reads and writes.  Sizes: N = n_tok, L = n_layers,
 * B = requests; device pointers unless marked host. */
typedef struct kvb_link_desc {
  int32_t mode;           /* KVB_LINK_CACHESLIDE, KVB_LINK_STATIC or KVB_LINK_CACHEBLEND */
  int32_t B, n_tok, n_layers, n_pages, vocab;
  int32_t rows;           /* row bound of layers 2..L: the sum of the per-request k
                           * (CacheSlide, CacheBlend), or the size of the static row set */
  int32_t period;         /* CacheSlide: refresh after layer l when l % period == 0 and l < L */
  int32_t refresh_rule;   /* KVB_REFRESH_LITERAL or KVB_REFRESH_DISSIM */
  int32_t alpha_mode;     /* CacheSlide fusion of layers 2..L: KVB_ALPHA_LAG / _CURRENT / _ONE */
  float tau;              /* refresh threshold */
  float scale;            /* attention scale, 1 / sqrt(hd) */
  const kvb_layer_weights* layers;     /* host [L] */
  const void* embedding;               /* [vocab, d] */
  const int32_t* tokens;               /* [N] vocabulary ids */
  const int32_t* pos;                  /* [N] RoPE positions in the spliced requests */
  const int32_t* lo;                   /* [N] first visible key (start of the request) */
  const int32_t* cu_tok;               /* [B + 1] */
  const int32_t* k_cap;                /* [B] k per request (CacheSlide, CacheBlend; NULL for static) */
  const int32_t* reuse_slot;           /* [L, N] slot of each token's compiled K/V, or -1 */
  const int32_t* const* new_pages;     /* host [L]: layer l + 1's new page ids (device) */
  const int32_t* const* cu_pages;      /* host [L]: its per-request offsets [B + 1] (device) */
  const int32_t* static_rows;          /* static: [rows] tokens, ascending within a request */
  const int32_t* static_cu;            /* static: [B + 1] row offsets of the requests */
  int32_t* page_table;                 /* [L, N] out: slot of every token's K/V per layer */
  void* k_pool;                        /* [n_pages, Hkv, 16, hd] in/out */
  void* v_pool;
  void* hidden;                        /* [N, d] out: hidden rows of the recomputed tokens */
  void* q;                             /* [N, Hq, hd] scratch */
  void* k;                             /* [N, Hkv, hd] scratch */
  void* v;                             /* [N, Hkv, hd] scratch */
  void* o;                             /* [N, Hq hd] scratch */
  float* d;                            /* [N] layer-1 deviation (CacheBlend: attention-map deviation) */
  float* alpha;                        /* [N] CacheSlide fusion weights */
  float* dev;                          /* [rows] per-row deviation of the current layer */
  float* cksim;                        /* [rows] per-row cosine similarity of a refresh layer */
  int32_t* ranking;                    /* [N] */
  int32_t* s_count;                    /* [B] */
  int32_t* cursor;                     /* [B] */
  int32_t* sel[2];                     /* [N] each: the selection, ping-pong across refreshes */
  int32_t* cu_rows[2];                 /* [B + 1] each */
  int32_t* dst_slot;                   /* [N] scratch */
  int32_t* page_dirty;                 /* [n_pages] SLIDE dirty counters, cleared here; or NULL */
  void* ws;                            /* workspace of kvb_workspace_size(max_rows >= N, max_tokens >= N, B) */
  size_t ws_bytes;
} kvb_link_desc;

/* The whole link step as one call: the layer loop of CacheSlide's Algorithm 2
 * (CacheSlide page, "Method details" and Algorithm 2: layer 1 recomputes
 * every token, the deviation ranks them and the top-k are recomputed in
 * layers 2..L, fused with the cached K/V, with the cosine refresh every
 * `period` layers), of EPIC's LegoLink (EPIC page, section 4: the static
 * set recomputed in every layer) or of the CacheBlend baseline as the EPIC
 * page describes it (section 3.2: layer 1 in full, kvb_attnmap_deviation and
 * kvb_topk, the selected rows replace the cached K/V in layers 2..L),
 * built from the calls above in the order a
 * caller would make them: per layer kvb_slot_map, kvb_qkv_fused (layer 1
 * batch-invariant, later layers allowed to split K), the refresh right after
 * the fusion when the layer has one, kvb_sparse_query_attn, kvb_mlp.
 * Nothing is read back to the host: every selective layer is launched for
 * link->rows rows and the device row counts bound the work, so the call
 * queues the step without a host synchronisation and can be recorded in a
 * HIP graph (the counters are cleared by a kernel, not a memset).  Results
 * are bitwise those of the same calls made one by one with these bounds.
 * *final_sel (host, may be NULL) receives which selection buffer holds the
 * set after the last layer.  Every argument is checked before anything is
 * queued; a HIP launch error returns KVB_ERR_HIP with the earlier steps
 * already queued. */
kvb_status kvb_link_run(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, const kvb_link_desc* link,
                        int32_t* final_sel);

#ifdef __cplusplus
}
#endif

#endif /* KVB_H */
