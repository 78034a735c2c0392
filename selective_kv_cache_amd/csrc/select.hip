// Top-k selection and the similarity-gated refresh of CacheSlide's Weighted
// Correction Attention (CacheSlide page, Algorithm 2).
//
// Ranking.  Each token gets the 64-bit key (~bits(d) << 32) | g.  For d >= 0
// the float bit pattern grows with d, so ascending keys list tokens by d
// descending, ties by lower index; d == 0 tokens come last.  Keys are unique.
//   1. chunk_sort: every request's token range is cut into 2048-key chunks,
//      each sorted in LDS with a bitonic network;
//   2. rank: a token's rank inside its request is the sum over the request's
//      chunks of the number of keys below its own (binary search), which gives
//      ranking[] directly and the top-k flag (rank < k_cap and d > 0);
//   3. compact: per request, an ordered scan of the flags writes the selected
//      tokens in ascending order and the row offsets.
// All steps are integer work on unique keys: the result is bitwise
// deterministic and independent of launch shapes.
#include "common.h"

#include <mutex>

namespace kvb {

template <class T>
kvb_status launch_deviation(hipStream_t st, int n_tok, const void* k_rec, const void* k_pool, int n_pages,
                            const int32_t* reuse_slot, float* d, float* alpha, int Hkv, int hd);

constexpr int CHUNK = 2048;
constexpr int SORT_THREADS = 1024;

__device__ __forceinline__ uint64_t make_key(float d, int g) {
  return ((uint64_t)(~__float_as_uint(d)) << 32) | (uint32_t)g;
}

// find the request of work item w when request b owns cdiv(N_b, CHUNK) chunks
__device__ __forceinline__ bool chunk_of(int w, int B, const int32_t* cu_tok, int* b_out, int* m_out) {
  for (int b = 0; b < B; b++) {
    const int n = cu_tok[b + 1] - cu_tok[b];
    const int nch = (n + CHUNK - 1) / CHUNK;
    if (w < nch) {
      *b_out = b;
      *m_out = w;
      return true;
    }
    w -= nch;
  }
  return false;
}

__global__ void __launch_bounds__(SORT_THREADS) chunk_sort_kernel(int B, const int32_t* __restrict__ cu_tok,
                                                                  const float* __restrict__ d,
                                                                  uint64_t* __restrict__ sorted) {
  __shared__ uint64_t keys[CHUNK];
  int b, m;
  if (!chunk_of(blockIdx.x, B, cu_tok, &b, &m)) return;
  const int s0 = cu_tok[b] + m * CHUNK;
  const int s1 = min(s0 + CHUNK, cu_tok[b + 1]);
  const int n = s1 - s0;
  for (int i = threadIdx.x; i < CHUNK; i += SORT_THREADS)
    keys[i] = i < n ? make_key(d[s0 + i], s0 + i) : ~0ull;
  __syncthreads();
  for (int k = 2; k <= CHUNK; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < CHUNK; i += SORT_THREADS) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t a = keys[i], c = keys[p];
          const bool up = (i & k) == 0;
          if ((a > c) == up) {
            keys[i] = c;
            keys[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < n; i += SORT_THREADS) sorted[s0 + i] = keys[i];
}

__global__ void rank_kernel(int B, int n_tok, const int32_t* __restrict__ cu_tok, const float* __restrict__ d,
                            const uint64_t* __restrict__ sorted, const int32_t* __restrict__ k_cap,
                            int32_t* __restrict__ ranking, int32_t* __restrict__ flag) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_tok) return;
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_tok[mid] <= g) lo = mid;
    else hi = mid;
  }
  const int b = lo, t0 = cu_tok[b], t1 = cu_tok[b + 1];
  if (g < t0 || g >= t1) return;
  const float dv = d[g];
  const uint64_t key = make_key(dv, g);
  int rank = 0;
  for (int s = t0; s < t1; s += CHUNK) {
    const int e = min(s + CHUNK, t1);
    int a = s, c = e;  // first index with sorted[idx] >= key
    while (a < c) {
      const int mid = (a + c) >> 1;
      if (sorted[mid] < key) a = mid + 1;
      else c = mid;
    }
    rank += a - s;
  }
  ranking[t0 + rank] = g;
  flag[g] = (rank < k_cap[b] && dv > 0.f) ? 1 : 0;
}

// Ordered compaction of flag[] per request: one block per request.  Each block
// first counts the flags of all earlier requests (its output offset), then
// scans its own range.  Writes out[offset + i], cu_rows[b+1], and optionally
// count_out[b] and s_count[b] = #{d > 0}.
constexpr int CT = 1024;

__device__ __forceinline__ int block_sum_int(int v, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int s = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); i++) s += sh[i];
  return s;
}

__global__ void __launch_bounds__(CT) compact_kernel(int B, const int32_t* __restrict__ cu_tok,
                                                     const int32_t* __restrict__ flag, int32_t* __restrict__ out,
                                                     int32_t* __restrict__ cu_rows, int32_t* __restrict__ count_out,
                                                     const float* __restrict__ d, int32_t* __restrict__ s_count) {
  __shared__ int sh[CT / 64];
  const int b = blockIdx.x;
  const int t0 = cu_tok[b], t1 = cu_tok[b + 1];
  int c = 0;
  for (int g = cu_tok[0] + threadIdx.x; g < t0; g += CT) c += flag[g];
  const int offset = block_sum_int(c, sh);
  int own = 0, pos = 0;
  for (int g = t0 + threadIdx.x; g < t1; g += CT) {
    own += flag[g];
    if (d) pos += d[g] > 0.f ? 1 : 0;
  }
  const int total = block_sum_int(own, sh);
  const int npos = d ? block_sum_int(pos, sh) : 0;
  if (threadIdx.x == 0) {
    if (b == 0) cu_rows[0] = 0;
    cu_rows[b + 1] = offset + total;
    if (count_out) count_out[b] = total;
    if (s_count) s_count[b] = npos;
  }
  // ordered scan over tiles of CT tokens: wave ballots + a per-tile wave prefix
  __shared__ int wsum[CT / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int base = offset;
  for (int s = t0; s < t1; s += CT) {
    const int g = s + threadIdx.x;
    const int f = (g < t1) ? flag[g] : 0;
    const uint64_t mask = __ballot(f);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wv] = __popcll(mask);
    __syncthreads();
    int woff = 0, tile_total = 0;
    for (int i = 0; i < CT / 64; i++) {
      if (i < wv) woff += wsum[i];
      tile_total += wsum[i];
    }
    if (f) out[base + woff + before] = g;
    __syncthreads();
    base += tile_total;
  }
}

// Refresh flags: one block per request.  Clears the request's flags, marks the
// kept rows, counts the retirees, marks the refills from the ranking and
// advances the cursor.
__global__ void __launch_bounds__(CT) refresh_flag_kernel(int B, const int32_t* __restrict__ cu_tok,
                                                          const int32_t* __restrict__ cu_rows_in,
                                                          const int32_t* __restrict__ sel_in,
                                                          const float* __restrict__ cksim, float tau, int rule,
                                                          const int32_t* __restrict__ ranking,
                                                          const int32_t* __restrict__ s_count,
                                                          int32_t* __restrict__ cursor, int32_t* __restrict__ flag) {
  __shared__ int sh[CT / 64];
  const int b = blockIdx.x;
  const int t0 = cu_tok[b], t1 = cu_tok[b + 1];
  for (int g = t0 + threadIdx.x; g < t1; g += CT) flag[g] = 0;
  __syncthreads();
  const int r0 = cu_rows_in[b], r1 = cu_rows_in[b + 1];
  int nret = 0;
  for (int r = r0 + threadIdx.x; r < r1; r += CT) {
    const float c = cksim[r];
    const bool retire = (rule == KVB_REFRESH_LITERAL) ? (c < tau) : (c > 1.f - tau);
    if (retire) nret++;
    else {
      const int g = sel_in[r];
      if (g >= t0 && g < t1) flag[g] = 1;
    }
  }
  const int R = block_sum_int(nret, sh);
  const int cur = cursor[b];
  const int avail = max(0, s_count[b] - cur);
  const int m = min(R, avail);
  for (int i = threadIdx.x; i < m; i += CT) {
    const int g = ranking[t0 + cur + i];
    if (g >= t0 && g < t1) flag[g] = 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) cursor[b] = cur + m;
}

struct TopkWs {
  uint64_t* sorted;
  int32_t* flag;
  int32_t* counts;
};

static TopkWs topk_ws(void* ws, int n_tok) {
  TopkWs w;
  char* p = (char*)ws;
  w.sorted = (uint64_t*)p;
  p += align_up((size_t)n_tok * 8 + CHUNK * 8, 256);
  w.flag = (int32_t*)p;
  p += align_up((size_t)n_tok * 4, 256);
  w.counts = (int32_t*)p;
  return w;
}

// sort, rank and compact of the per-request top-k by d (d already written)
static kvb_status launch_topk(hipStream_t st, int B, int n_tok, const int32_t* cu_tok, const float* d,
                              const int32_t* k_cap, int32_t* ranking, int32_t* s_count, int32_t* sel,
                              int32_t* cu_rows, int32_t* cursor, void* ws) {
  TopkWs w = topk_ws(ws, n_tok);
  if (n_tok > 0) {
    const int n_chunks = n_tok / CHUNK + B;  // >= sum over requests of cdiv(N_b, CHUNK)
    {
      LaunchTimer lt(st, "topk_sort");
      chunk_sort_kernel<<<n_chunks, SORT_THREADS, 0, st>>>(B, cu_tok, d, w.sorted);
    }
    KVB_TRY(check_launch("chunk_sort_kernel"));
    {
      LaunchTimer lt(st, "topk_rank");
      rank_kernel<<<cdiv(n_tok, 256), 256, 0, st>>>(B, n_tok, cu_tok, d, w.sorted, k_cap, ranking, w.flag);
    }
    KVB_TRY(check_launch("rank_kernel"));
  }
  {
    LaunchTimer lt(st, "topk_compact");
    compact_kernel<<<B, CT, 0, st>>>(B, cu_tok, w.flag, sel, cu_rows, cursor, d, s_count);
  }
  return check_launch("compact_kernel");
}

// ------------------------------------------------ allocation-free top-k scratch
// kvb_deviation_topk_noalloc keeps the top-k keys and flags in this fixed
// array instead of a caller workspace.  Each GPU holds its own copy until the
// process ends; host code takes its device address from hipGetSymbolAddress
// (the array's name is not a device address on the host) and keeps it per
// device.  The sorted keys and flags are always written before they are read,
// so nothing in it needs clearing between calls.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)2 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// Device address of this device's scratch (the device is current).  The first
// call on a device looks it up; later calls return the kept pointer.
kvb_status noalloc_scratch(int device, void** out) {
  if (device < 0 || device >= NOALLOC_MAX_DEVICES) return fail(KVB_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVB_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return KVB_OK;
}

// Called by kvb_create with `device` current, so the lookup happens at set-up.
kvb_status noalloc_scratch_setup(int device) {
  void* p = nullptr;
  return noalloc_scratch(device, &p);
}

static kvb_status check_deviation_topk(const kvb_model_desc* desc, int32_t B, int32_t n_tok, const int32_t* cu_tok,
                                       const void* k_rec, const void* k_pool, int32_t n_pages,
                                       const int32_t* reuse_slot, const int32_t* k_cap, float* d, float* alpha,
                                       int32_t* ranking, int32_t* s_count, int32_t* sel, int32_t* cu_rows,
                                       int32_t* cursor) {
  KVB_TRY(check_desc(desc));
  if (B <= 0 || n_tok < 0 || n_pages < 0) return fail(KVB_ERR_INVALID_ARG, "B <= 0 or negative size");
  KVB_CHECK_PTR(cu_tok, "cu_tok");
  KVB_CHECK_PTR(k_cap, "k_cap");
  KVB_CHECK_PTR(s_count, "s_count");
  KVB_CHECK_PTR(cu_rows, "cu_rows");
  KVB_CHECK_PTR(cursor, "cursor");
  if (n_tok > 0) {
    KVB_CHECK_PTR(k_rec, "k_rec");
    KVB_CHECK_PTR(k_pool, "k_pool");
    KVB_CHECK_PTR(reuse_slot, "reuse_slot");
    KVB_CHECK_PTR(d, "d");
    KVB_CHECK_PTR(alpha, "alpha");
    KVB_CHECK_PTR(ranking, "ranking");
    KVB_CHECK_PTR(sel, "sel");
  }
  if (desc->n_kv_heads * desc->head_dim / 8 > 1024) return fail(KVB_ERR_UNSUPPORTED, "n_kv_heads * head_dim > 8192");
  return KVB_OK;
}

static kvb_status run_deviation_topk(hipStream_t st, const kvb_model_desc* desc, int32_t B, int32_t n_tok,
                                     const int32_t* cu_tok, const void* k_rec, const void* k_pool, int32_t n_pages,
                                     const int32_t* reuse_slot, const int32_t* k_cap, float* d, float* alpha,
                                     int32_t* ranking, int32_t* s_count, int32_t* sel, int32_t* cu_rows,
                                     int32_t* cursor, void* ws) {
  if (desc->dtype == KVB_BF16)
    KVB_TRY(launch_deviation<bf16_t>(st, n_tok, k_rec, k_pool, n_pages, reuse_slot, d, alpha, desc->n_kv_heads,
                                     desc->head_dim));
  else
    KVB_TRY(launch_deviation<float>(st, n_tok, k_rec, k_pool, n_pages, reuse_slot, d, alpha, desc->n_kv_heads,
                                    desc->head_dim));
  return launch_topk(st, B, n_tok, cu_tok, d, k_cap, ranking, s_count, sel, cu_rows, cursor, ws);
}

}  // namespace kvb

using namespace kvb;

extern "C" kvb_status kvb_topk(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B, int32_t n_tok,
                               const int32_t* cu_tok, const float* d, const int32_t* k_cap, int32_t* ranking,
                               int32_t* s_count, int32_t* sel, int32_t* cu_rows, int32_t* cursor, void* ws,
                               size_t ws_bytes) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (B <= 0 || n_tok < 0) return fail(KVB_ERR_INVALID_ARG, "B <= 0 or negative size");
  KVB_CHECK_PTR(cu_tok, "cu_tok");
  KVB_CHECK_PTR(k_cap, "k_cap");
  KVB_CHECK_PTR(s_count, "s_count");
  KVB_CHECK_PTR(cu_rows, "cu_rows");
  KVB_CHECK_PTR(cursor, "cursor");
  if (n_tok > 0) {
    KVB_CHECK_PTR(d, "d");
    KVB_CHECK_PTR(ranking, "ranking");
    KVB_CHECK_PTR(sel, "sel");
  }
  if (!ws || ws_bytes < ws_topk_bytes(n_tok, B)) return fail(KVB_ERR_WORKSPACE, "kvb_topk workspace too small");
  CtxScope scope(ctx);
  return launch_topk((hipStream_t)stream, B, n_tok, cu_tok, d, k_cap, ranking, s_count, sel, cu_rows, cursor, ws);
}

extern "C" kvb_status kvb_deviation_topk(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B,
                                         int32_t n_tok, const int32_t* cu_tok, const void* k_rec, const void* k_pool,
                                         int32_t n_pages, const int32_t* reuse_slot, const int32_t* k_cap, float* d,
                                         float* alpha, int32_t* ranking, int32_t* s_count, int32_t* sel,
                                         int32_t* cu_rows, int32_t* cursor, void* ws, size_t ws_bytes) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_deviation_topk(desc, B, n_tok, cu_tok, k_rec, k_pool, n_pages, reuse_slot, k_cap, d, alpha, ranking,
                               s_count, sel, cu_rows, cursor));
  if (!ws || ws_bytes < ws_topk_bytes(n_tok, B)) return fail(KVB_ERR_WORKSPACE, "kvb_deviation_topk workspace too small");
  CtxScope scope(ctx);
  return run_deviation_topk((hipStream_t)stream, desc, B, n_tok, cu_tok, k_rec, k_pool, n_pages, reuse_slot, k_cap,
                            d, alpha, ranking, s_count, sel, cu_rows, cursor, ws);
}

extern "C" kvb_status kvb_deviation_topk_noalloc(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B,
                                                 int32_t n_tok, const int32_t* cu_tok, const void* k_rec,
                                                 const void* k_pool, int32_t n_pages, const int32_t* reuse_slot,
                                                 const int32_t* k_cap, float* d, float* alpha, int32_t* ranking,
                                                 int32_t* s_count, int32_t* sel, int32_t* cu_rows, int32_t* cursor) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_deviation_topk(desc, B, n_tok, cu_tok, k_rec, k_pool, n_pages, reuse_slot, k_cap, d, alpha, ranking,
                               s_count, sel, cu_rows, cursor));
  if (n_tok > KVB_NOALLOC_MAX_TOKENS || B > KVB_NOALLOC_MAX_REQUESTS ||
      ws_topk_bytes(n_tok, B) > NOALLOC_SCRATCH_BYTES)
    return fail(KVB_ERR_WORKSPACE, "kvb_deviation_topk_noalloc: more than " + std::to_string(KVB_NOALLOC_MAX_TOKENS) +
                                       " tokens or " + std::to_string(KVB_NOALLOC_MAX_REQUESTS) +
                                       " requests for its fixed scratch");
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  void* ws = nullptr;
  KVB_TRY(noalloc_scratch(dev, &ws));
  CtxScope scope(ctx);
  return run_deviation_topk((hipStream_t)stream, desc, B, n_tok, cu_tok, k_rec, k_pool, n_pages, reuse_slot, k_cap,
                            d, alpha, ranking, s_count, sel, cu_rows, cursor, ws);
}

extern "C" kvb_status kvb_cosine_refresh(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B,
                                         int32_t n_tok, const int32_t* cu_tok, int32_t T_max,
                                         const int32_t* cu_rows_in, const int32_t* sel_in, const float* cksim,
                                         float tau, int32_t rule, const int32_t* ranking, const int32_t* s_count,
                                         int32_t* cursor, int32_t* sel_out, int32_t* cu_rows_out, void* ws,
                                         size_t ws_bytes) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (B <= 0 || n_tok < 0 || T_max < 0) return fail(KVB_ERR_INVALID_ARG, "B <= 0 or negative size");
  if (rule != KVB_REFRESH_LITERAL && rule != KVB_REFRESH_DISSIM) return fail(KVB_ERR_INVALID_ARG, "bad rule");
  KVB_CHECK_PTR(cu_tok, "cu_tok");
  KVB_CHECK_PTR(cu_rows_in, "cu_rows_in");
  KVB_CHECK_PTR(cu_rows_out, "cu_rows_out");
  KVB_CHECK_PTR(ranking, "ranking");
  KVB_CHECK_PTR(s_count, "s_count");
  KVB_CHECK_PTR(cursor, "cursor");
  KVB_CHECK_PTR(sel_out, "sel_out");
  if (T_max > 0) {
    KVB_CHECK_PTR(sel_in, "sel_in");
    KVB_CHECK_PTR(cksim, "cksim");
  }
  if (sel_in && sel_in == sel_out) return fail(KVB_ERR_INVALID_ARG, "sel_in and sel_out must not overlap");
  if (!ws || ws_bytes < ws_refresh_bytes(n_tok, B)) return fail(KVB_ERR_WORKSPACE, "kvb_cosine_refresh workspace too small");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  int32_t* flag = (int32_t*)ws;
  {
    LaunchTimer lt(st, "refresh_flag");
    refresh_flag_kernel<<<B, CT, 0, st>>>(B, cu_tok, cu_rows_in, sel_in, cksim, tau, rule, ranking, s_count, cursor,
                                          flag);
  }
  KVB_TRY(check_launch("refresh_flag_kernel"));
  {
    LaunchTimer lt(st, "refresh_compact");
    compact_kernel<<<B, CT, 0, st>>>(B, cu_tok, flag, sel_out, cu_rows_out, nullptr, nullptr, nullptr);
  }
  return check_launch("compact_kernel");
}
