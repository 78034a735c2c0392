// Internal helpers shared by the kvb HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <string.h>
#include <math.h>

#include <string>
#include <vector>

#include "../../include/kvb.h"

// ------------------------------------------------------------------ errors

namespace kvb {

void set_error(const std::string& msg);
kvb_status fail(kvb_status s, const std::string& msg);
kvb_status check_launch(const char* what);

// Per-context launch timing (tracing): when enabled, kernels whose name
// contains the filter string are bracketed with HIP events on their stream.
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
struct Ctx {
  int device = 0;
  int n_cu = 256;
  bool timing = false;
  std::string filter;
  std::vector<TimingRec> recs;
  std::vector<hipEvent_t> spare;
  std::vector<std::string> pend_names;  // totals not yet read by kvb_timing_read
  std::vector<double> pend_ms;
  std::vector<long> pend_count;
};

// The context of the entry point running on this thread (set by CtxScope).
Ctx* current_ctx();
struct CtxScope {
  Ctx* prev;
  explicit CtxScope(kvb_ctx* c);
  ~CtxScope();
};

// Bracket one kernel launch with timing events when the current context asks
// for it.  By default the events are recorded on the stream before and after
// the launch; with `ext` the launch itself records them (start and stop of
// the dispatch, hipExtLaunchKernelGGL with start() and stop()), which puts no
// marker between this kernel and its neighbours.
struct LaunchTimer {
  Ctx* c = nullptr;
  hipStream_t st;
  const char* name;
  hipEvent_t a = nullptr, b = nullptr;
  bool ext;
  LaunchTimer(hipStream_t s, const char* n, bool ext = false);
  ~LaunchTimer();
  hipEvent_t start() const { return ext ? a : nullptr; }
  hipEvent_t stop() const { return ext ? b : nullptr; }
};

// Validates the model description; returns KVB_OK or an error with message.
kvb_status check_desc(const kvb_model_desc* d);
kvb_status check_ctx(const kvb_ctx* c);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// Device address of this device's fixed scratch of the allocation-free top-k
// (first call on a device looks it up); setup is called by kvb_create.
kvb_status noalloc_scratch(int device, void** out);
kvb_status noalloc_scratch_setup(int device);

// workspace layouts (bytes), shared by kvb_workspace_size and the entry points
size_t ws_mlp_bytes(const kvb_model_desc* d, int32_t max_rows, int n_cu);
size_t ws_gemm_sk_bytes(int n_cu);
size_t ws_qkv_bytes(const kvb_model_desc* d, int32_t max_rows);

// One bf16 row on a split-K launch, nothing fused with a cached row: RMSNorm,
// the one-row Q/K/V product, and in its epilogue RoPE of Q and K and the K/V
// store into slot dst_slot[0] (what kvb_qkv_proj without RoPE followed by the
// RoPE + fusion pass in KVB_ALPHA_ONE mode writes, bitwise).
kvb_status qkv_rope_one_row(hipStream_t st, const kvb_model_desc* d, const int32_t* n_rows, const int32_t* row_tok,
                            const void* hidden, const void* norm_w, const void* w_qkv, const int32_t* tok_pos, void* q,
                            void* k, void* v, void* k_pool, void* v_pool, int n_slots, const int32_t* dst_slot,
                            void* ws);
size_t ws_topk_bytes(int32_t max_tokens, int32_t max_requests);
size_t ws_refresh_bytes(int32_t max_tokens, int32_t max_requests);
size_t ws_attn_bytes(const kvb_model_desc* d, int32_t max_rows, int n_cu);
size_t ws_attnmap_bytes(const kvb_model_desc* d, int32_t max_tokens);

}  // namespace kvb

#define KVB_CHECK_PTR(p, name) \
  do { if (!(p)) return kvb::fail(KVB_ERR_INVALID_ARG, std::string(name) + " is NULL"); } while (0)
#define KVB_TRY(expr) \
  do { kvb_status _s = (expr); if (_s != KVB_OK) return _s; } while (0)

// ------------------------------------------------------------------ bf16

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bfloat16, round to nearest even (gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// storage-type traits: T is float (KVB_F32) or bf16_t (KVB_BF16)
template <class T> struct Store;
template <> struct Store<float> {
  __device__ __forceinline__ static float ld(const float* p) { return *p; }
  __device__ __forceinline__ static void st(float* p, float v) { *p = v; }
  __device__ __forceinline__ static float cvt(float v) { return v; }
};
template <> struct Store<bf16_t> {
  __device__ __forceinline__ static float ld(const bf16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static void st(bf16_t* p, float v) { *p = f2bf(v); }
  __device__ __forceinline__ static bf16_t cvt(float v) { return f2bf(v); }
};

template <class T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

__device__ __forceinline__ int cdiv_dev(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ int row_count(const int32_t* n_rows, int T_max) {
  if (!n_rows) return T_max;
  int n = *n_rows;
  return n < T_max ? n : T_max;
}

// ---- direct-to-LDS loads (gfx950 global_load_lds_*), issued as inline
// assembly so that the compiler, which cannot tell which LDS bytes such a load
// writes, does not drain every outstanding load before each LDS read.  The
// LDS base must be wave-uniform; completion is tracked with explicit vmcnt
// waits before the barrier that publishes the data.

// 16 bytes per lane from g, landing at LDS address lds_base + 16 * lane
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base) : "memory");
}

// 4 bytes per lane from g, landing at LDS address lds_base + 4 * lane
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_base) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");  // LDS reads of the loaded data stay after the wait
}

// workgroup barrier that orders LDS accesses without draining outstanding
// global (and LDS-DMA) loads, unlike __syncthreads: this wave's LDS reads and
// writes complete (lgkmcnt 0) before it arrives
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, b2_t));
}

// slot s of head h in a K or V pool laid out [page][head][16][hd]
__device__ __forceinline__ size_t pool_off(int slot, int h, int Hkv, int hd) {
  return (((size_t)(slot >> 4) * Hkv + h) * 16 + (slot & 15)) * hd;
}

// CacheSlide's correction weight d / ||K_reuse||^2 (0 if both are 0, 1 if
// only the norm is 0)
__device__ __forceinline__ float alpha_rule(float d, float nrm) {
  if (nrm > 0.f) return d / nrm;
  return d == 0.f ? 0.f : 1.f;
}

// Rotate-half RoPE frequencies base^(-2j/hd), j < hd / 2, in double precision,
// formed on the host and passed to the kernels by value.
struct RopeFreq {
  double f[64];
};

inline RopeFreq rope_freq(int hd, float base) {
  RopeFreq rf{};
  for (int j = 0; j < hd / 2 && j < 64; j++) rf.f[j] = exp2(-2.0 * (double)j / (double)hd * log2((double)base));
  return rf;
}

// cosine and sine of the angle pos * f: formed and reduced to [-pi, pi] in
// double precision, then sincos in float
__device__ __forceinline__ float2 rope_cs(int pos, double f) {
  const double a = (double)pos * f;
  const double twopi = 6.283185307179586;
  const double red = fma(-rint(a / twopi), twopi, a);
  float s, c;
  sincosf((float)red, &s, &c);
  return make_float2(c, s);
}

// the two halves of a rotated pair, with the products and their one fused
// add spelled out so that every kernel rounds them the same way
__device__ __forceinline__ float rot_lo(float x1, float x2, float c, float s) { return fmaf(x1, c, -(x2 * s)); }
__device__ __forceinline__ float rot_hi(float x2, float x1, float c, float s) { return fmaf(x2, c, x1 * s); }

// wave64 reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
