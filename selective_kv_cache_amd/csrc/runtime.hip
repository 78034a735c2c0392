// Host runtime of the kvb library: status strings, thread-local errors,
// context, argument checks, workspace sizing and the deterministic page
// allocator (lowest free id first, SLIDE's preallocated new pages).
#include <algorithm>
#include <cstdio>
#include <set>
#include <string>
#include <vector>

#include "common.h"

namespace kvb {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

kvb_status fail(kvb_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

kvb_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return KVB_OK;
}

static thread_local Ctx* g_current = nullptr;

Ctx* current_ctx() { return g_current; }

CtxScope::CtxScope(kvb_ctx* c) : prev(g_current) { g_current = reinterpret_cast<Ctx*>(c); }
CtxScope::~CtxScope() { g_current = prev; }

static hipEvent_t take_event(Ctx* c) {
  if (!c->spare.empty()) {
    hipEvent_t e = c->spare.back();
    c->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

LaunchTimer::LaunchTimer(hipStream_t s, const char* n, bool e) : st(s), name(n), ext(e) {
  Ctx* cur = g_current;
  if (!cur || !cur->timing) return;
  if (!cur->filter.empty() && std::string(n).find(cur->filter) == std::string::npos) return;
  a = take_event(cur);
  if (!a) return;
  if (ext) {
    // both events go to the launch, which records them
    b = take_event(cur);
    if (!b) {
      cur->spare.push_back(a);
      a = nullptr;
      return;
    }
    c = cur;
    return;
  }
  if (hipEventRecord(a, st) != hipSuccess) {
    cur->spare.push_back(a);
    a = nullptr;
    return;
  }
  c = cur;
}

LaunchTimer::~LaunchTimer() {
  if (!c) return;
  if (!ext) {
    b = take_event(c);
    if (!b || hipEventRecord(b, st) != hipSuccess) {
      c->spare.push_back(a);
      if (b) c->spare.push_back(b);
      return;
    }
  }
  c->recs.push_back(TimingRec{name, a, b});
}

kvb_status check_ctx(const kvb_ctx* c) {
  if (!c) return fail(KVB_ERR_INVALID_ARG, "ctx is NULL");
  return KVB_OK;
}

kvb_status check_desc(const kvb_model_desc* d) {
  if (!d) return fail(KVB_ERR_INVALID_ARG, "desc is NULL");
  if (d->d_model <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->ffn <= 0)
    return fail(KVB_ERR_INVALID_ARG, "model sizes must be positive");
  if (d->n_kv_heads > 64) return fail(KVB_ERR_UNSUPPORTED, "n_kv_heads must be <= 64");
  if (d->n_q_heads % d->n_kv_heads)
    return fail(KVB_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KVB_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->page_size != 16) return fail(KVB_ERR_UNSUPPORTED, "page_size must be 16");
  if (d->dtype != KVB_F32 && d->dtype != KVB_BF16) return fail(KVB_ERR_UNSUPPORTED, "dtype must be KVB_F32 or KVB_BF16");
  if (!(d->rms_eps >= 0.f) || !(d->rope_base > 0.f)) return fail(KVB_ERR_INVALID_ARG, "rms_eps / rope_base out of range");
  if (d->dtype == KVB_BF16) {
    if (d->d_model % 64 || d->ffn % 64 || (d->n_q_heads * d->head_dim) % 64)
      return fail(KVB_ERR_UNSUPPORTED, "bf16 path needs d_model, ffn and n_q_heads*head_dim to be multiples of 64");
  }
  return KVB_OK;
}

static size_t esize(const kvb_model_desc* d) { return d->dtype == KVB_BF16 ? 2 : 4; }

size_t ws_mlp_bytes(const kvb_model_desc* d, int32_t max_rows, int n_cu) {
  // h1 [T, d] and u [T, F] in storage type; bf16 adds the normalised h1 [T, d]
  // and the stream-K partials of its products
  return align_up((size_t)max_rows * d->d_model * esize(d), 256) +
         align_up((size_t)max_rows * d->ffn * esize(d), 256) + ws_qkv_bytes(d, max_rows) +
         (d->dtype == KVB_BF16 ? ws_gemm_sk_bytes(n_cu) : 0);
}

size_t ws_qkv_bytes(const kvb_model_desc* d, int32_t max_rows) {
  // bf16: the normalised rows [T, d]; float32 normalises inside the GEMM
  return d->dtype == KVB_BF16 ? align_up((size_t)max_rows * d->d_model * 2, 256) : 0;
}

size_t ws_topk_bytes(int32_t max_tokens, int32_t max_requests) {
  // sorted keys u64 [n_tok + pad], rank/flag int32 [n_tok], counts int32 [2B + 2]
  size_t n = (size_t)max_tokens;
  return align_up(n * 8 + 2048 * 8, 256) + align_up(n * 4, 256) + align_up(((size_t)max_requests * 2 + 2) * 4, 256);
}

size_t ws_refresh_bytes(int32_t max_tokens, int32_t max_requests) {
  return align_up((size_t)max_tokens * 4, 256) + align_up(((size_t)max_requests * 2 + 2) * 4, 256);
}


}  // namespace kvb

using namespace kvb;

extern "C" {

const char* kvb_status_string(kvb_status s) {
  switch (s) {
    case KVB_OK: return "ok";
    case KVB_ERR_INVALID_ARG: return "invalid argument";
    case KVB_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVB_ERR_HIP: return "HIP error";
    case KVB_ERR_CAPACITY: return "page pool exhausted";
    case KVB_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* kvb_last_error(void) { return g_last_error.c_str(); }

kvb_status kvb_create(int32_t device, kvb_ctx** out) {
  if (!out) return fail(KVB_ERR_INVALID_ARG, "out is NULL");
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string("hipGetDeviceCount: ") + hipGetErrorString(e));
  if (device < 0 || device >= n) return fail(KVB_ERR_INVALID_ARG, "device index out of range");
  // with `device` current, look up the device address of the fixed scratch of
  // the allocation-free entry point once for this device
  int prev = 0;
  e = hipGetDevice(&prev);
  if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (prev != device && (e = hipSetDevice(device)) != hipSuccess)
    return fail(KVB_ERR_HIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
  const kvb_status s = noalloc_scratch_setup(device);
  if (prev != device) hipSetDevice(prev);
  if (s != KVB_OK) return s;
  Ctx* c = new Ctx();
  c->device = device;
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && cu > 0) c->n_cu = cu;
  *out = reinterpret_cast<kvb_ctx*>(c);
  return KVB_OK;
}

kvb_status kvb_destroy(kvb_ctx* ctx) {
  Ctx* c = reinterpret_cast<Ctx*>(ctx);
  if (c) {
    for (auto& r : c->recs) {
      hipEventDestroy(r.a);
      hipEventDestroy(r.b);
    }
    for (auto e : c->spare) hipEventDestroy(e);
  }
  delete c;
  return KVB_OK;
}

kvb_status kvb_timing_enable(kvb_ctx* ctx, const char* filter) {
  KVB_TRY(check_ctx(ctx));
  Ctx* c = reinterpret_cast<Ctx*>(ctx);
  c->timing = filter != nullptr;
  c->filter = filter ? filter : "";
  return KVB_OK;
}

kvb_status kvb_timing_read(kvb_ctx* ctx, char* buf, size_t len, size_t* needed) {
  KVB_TRY(check_ctx(ctx));
  Ctx* c = reinterpret_cast<Ctx*>(ctx);
  // fold the finished records into the pending per-name totals (first-seen order)
  for (auto& r : c->recs) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string("hipEventSynchronize: ") + hipGetErrorString(e));
    float t = 0.f;
    e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string("hipEventElapsedTime: ") + hipGetErrorString(e));
    size_t i = 0;
    while (i < c->pend_names.size() && c->pend_names[i] != r.name) i++;
    if (i == c->pend_names.size()) {
      c->pend_names.push_back(r.name);
      c->pend_ms.push_back(0.0);
      c->pend_count.push_back(0);
    }
    c->pend_ms[i] += t;
    c->pend_count[i] += 1;
    c->spare.push_back(r.a);
    c->spare.push_back(r.b);
  }
  c->recs.clear();
  std::string out = "{";
  for (size_t i = 0; i < c->pend_names.size(); i++) {
    char item[256];
    snprintf(item, sizeof item, "%s\"%s\": {\"count\": %ld, \"ms\": %.6f}", i ? ", " : "",
             c->pend_names[i].c_str(), c->pend_count[i], c->pend_ms[i]);
    out += item;
  }
  out += "}";
  if (needed) *needed = out.size() + 1;
  if (buf && len >= out.size() + 1) {
    memcpy(buf, out.c_str(), out.size() + 1);
    c->pend_names.clear();
    c->pend_ms.clear();
    c->pend_count.clear();
  }
  return KVB_OK;
}

kvb_status kvb_workspace_size(kvb_ctx* ctx, const kvb_model_desc* desc, int32_t max_rows, int32_t max_tokens,
                              int32_t max_requests, size_t* bytes) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  KVB_CHECK_PTR(bytes, "bytes");
  if (max_rows < 0 || max_tokens < 0 || max_requests < 0) return fail(KVB_ERR_INVALID_ARG, "negative size");
  size_t b = ws_mlp_bytes(desc, max_rows, reinterpret_cast<Ctx*>(ctx)->n_cu);
  b = std::max(b, ws_qkv_bytes(desc, max_rows) + (desc->dtype == KVB_BF16 ? ws_gemm_sk_bytes(0) : 0));
  b = std::max(b, ws_topk_bytes(max_tokens, max_requests));
  b = std::max(b, ws_refresh_bytes(max_tokens, max_requests));
  b = std::max(b, ws_attn_bytes(desc, max_rows, reinterpret_cast<Ctx*>(ctx)->n_cu));
  b = std::max(b, ws_attnmap_bytes(desc, max_tokens));
  *bytes = b;
  return KVB_OK;
}

// ------------------------------------------------------------ page allocator

struct kvb_pool {
  int32_t n_pages;
  std::set<int32_t> free_ids;
  std::vector<uint8_t> used;
};

kvb_status kvb_pool_create(int32_t n_pages, kvb_pool** out) {
  if (!out) return fail(KVB_ERR_INVALID_ARG, "out is NULL");
  if (n_pages < 0) return fail(KVB_ERR_INVALID_ARG, "n_pages < 0");
  kvb_pool* p = new kvb_pool();
  p->n_pages = n_pages;
  p->used.assign(n_pages, 0);
  for (int32_t i = 0; i < n_pages; i++) p->free_ids.insert(p->free_ids.end(), i);
  *out = p;
  return KVB_OK;
}

kvb_status kvb_pool_destroy(kvb_pool* pool) {
  delete pool;
  return KVB_OK;
}

kvb_status kvb_pool_alloc(kvb_pool* pool, int32_t n, int32_t* out_ids) {
  if (!pool) return fail(KVB_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0) return fail(KVB_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && !out_ids) return fail(KVB_ERR_INVALID_ARG, "out_ids is NULL");
  if ((size_t)n > pool->free_ids.size())
    return fail(KVB_ERR_CAPACITY, "page pool exhausted: need " + std::to_string(n) + ", free " +
                                      std::to_string(pool->free_ids.size()));
  auto it = pool->free_ids.begin();
  for (int32_t i = 0; i < n; i++) {
    out_ids[i] = *it;
    pool->used[*it] = 1;
    it = pool->free_ids.erase(it);
  }
  return KVB_OK;
}

kvb_status kvb_pool_release(kvb_pool* pool, int32_t n, const int32_t* ids) {
  if (!pool) return fail(KVB_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0) return fail(KVB_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && !ids) return fail(KVB_ERR_INVALID_ARG, "ids is NULL");
  for (int32_t i = 0; i < n; i++) {
    int32_t id = ids[i];
    if (id < 0 || id >= pool->n_pages || !pool->used[id])
      return fail(KVB_ERR_INVALID_ARG, "releasing page " + std::to_string(id) + " that is not allocated");
  }
  for (int32_t i = 0; i < n; i++) {
    pool->used[ids[i]] = 0;
    pool->free_ids.insert(ids[i]);
  }
  return KVB_OK;
}

kvb_status kvb_pool_free_count(const kvb_pool* pool, int32_t* out) {
  if (!pool || !out) return fail(KVB_ERR_INVALID_ARG, "pool or out is NULL");
  *out = (int32_t)pool->free_ids.size();
  return KVB_OK;
}

// ------------------------------------------------------------ page tiers

kvb_status kvb_pages_copy(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t direction,
                          const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int32_t* page_ids,
                          int32_t n_ids) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (direction != KVB_COPY_H2D && direction != KVB_COPY_D2H)
    return fail(KVB_ERR_INVALID_ARG, "direction must be KVB_COPY_H2D or KVB_COPY_D2H");
  if (n_ids < 0) return fail(KVB_ERR_INVALID_ARG, "n_ids < 0");
  if (n_ids == 0) return KVB_OK;
  if (!page_ids) return fail(KVB_ERR_INVALID_ARG, "page_ids is NULL");
  if (!src_k && dst_k) return fail(KVB_ERR_INVALID_ARG, "src_k is NULL");
  if (!src_v && dst_v) return fail(KVB_ERR_INVALID_ARG, "src_v is NULL");
  for (int32_t i = 0; i < n_ids; i++)
    if (page_ids[i] < 0) return fail(KVB_ERR_INVALID_ARG, "negative page id");
  CtxScope scope(ctx);
  const size_t esz = desc->dtype == KVB_BF16 ? 2 : 4;
  const size_t page_bytes = (size_t)desc->n_kv_heads * 16 * desc->head_dim * esz;
  const hipMemcpyKind kind = direction == KVB_COPY_H2D ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
  hipStream_t st = (hipStream_t)stream;
  // one copy per run of consecutive ids, for K then V
  int32_t i = 0;
  while (i < n_ids) {
    int32_t j = i + 1;
    while (j < n_ids && page_ids[j] == page_ids[j - 1] + 1) j++;
    const size_t off = (size_t)page_ids[i] * page_bytes, len = (size_t)(j - i) * page_bytes;
    if (dst_k) {
      const hipError_t e = hipMemcpyAsync((char*)dst_k + off, (const char*)src_k + off, len, kind, st);
      if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
    }
    if (dst_v) {
      const hipError_t e = hipMemcpyAsync((char*)dst_v + off, (const char*)src_v + off, len, kind, st);
      if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
    }
    i = j;
  }
  return KVB_OK;
}

}  // extern "C"
