// Bandwidth-bound row kernels of the link step: embedding gather, RoPE,
// CacheSlide's fusion + scatter into new pages, and the per-layer slot map.
//
// Every reduction here runs in a fixed order that depends only on the element
// index inside a row, never on the row's place in a batch, so results are
// bitwise reproducible from run to run and from batch to batch.
#include "common.h"

#include <type_traits>

#include <algorithm>

namespace kvb {

// ------------------------------------------------------------------ embedding
// hidden[g] = table[tokens[g]], g = row_tok[r]

template <class T>
__global__ void embed_kernel(int T_max, const int32_t* __restrict__ n_rows, const int32_t* __restrict__ row_tok,
                             const int32_t* __restrict__ tokens, int vocab, const T* __restrict__ table,
                             T* __restrict__ hidden, int d) {
  const int r = blockIdx.x;
  if (r >= row_count(n_rows, T_max)) return;
  const int g = row_tok ? row_tok[r] : r;
  const int id = tokens[g];
  if (id < 0 || id >= vocab) return;
  const uint4* src = reinterpret_cast<const uint4*>(table + (size_t)id * d);
  uint4* dst = reinterpret_cast<uint4*>(hidden + (size_t)g * d);
  const int nvec = d * (int)sizeof(T) / 16;
  for (int i = threadIdx.x; i < nvec; i += blockDim.x) dst[i] = src[i];
}

// ------------------------------------------------------------------ RoPE
// rotate-half: (x_j, x_{j+hd/2}) -> (x_j c - x_{j+hd/2} s, x_{j+hd/2} c + x_j s),
// angle = pos * base^(-2j/hd).  The angle is formed and reduced to [-pi, pi] in
// double precision; its cosine and sine are then taken in float.

template <class T> __device__ __forceinline__ void load8(const T* p, float* o);
template <class T> __device__ __forceinline__ void store8(T* p, const float* v);


template <class T>
__global__ void __launch_bounds__(256) rope_kernel(int T_max, const int32_t* __restrict__ n_rows,
                                                   const int32_t* __restrict__ row_tok,
                                                   const int32_t* __restrict__ tok_pos, T* __restrict__ q,
                                                   T* __restrict__ k, int Hq, int Hkv, int hd, RopeFreq rf) {
  const int r = blockIdx.x;
  if (r >= row_count(n_rows, T_max)) return;
  const int g = row_tok ? row_tok[r] : r;
  const int half = hd / 2;
  __shared__ float cs[64], sn[64];
  if (threadIdx.x < half) {
    const float2 c = rope_cs(tok_pos[g], rf.f[threadIdx.x]);
    cs[threadIdx.x] = c.x;
    sn[threadIdx.x] = c.y;
  }
  __syncthreads();
  // one item = 8 consecutive pairs (j .. j+7, j+half .. j+half+7) of one head
  const int gph = half / 8;
  const int items = (Hq + Hkv) * gph;
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int h = it / gph, j = (it % gph) * 8;
    T* x = (h < Hq) ? (q + ((size_t)r * Hq + h) * hd) : (k + ((size_t)r * Hkv + (h - Hq)) * hd);
    float x1[8], x2[8], y1[8], y2[8];
    load8<T>(x + j, x1);
    load8<T>(x + j + half, x2);
#pragma unroll
    for (int e = 0; e < 8; e++) {
      y1[e] = rot_lo(x1[e], x2[e], cs[j + e], sn[j + e]);
      y2[e] = rot_hi(x2[e], x1[e], cs[j + e], sn[j + e]);
    }
    store8<T>(x + j, y1);
    store8<T>(x + j + half, y2);
  }
}


// 8 consecutive elements of a row as float
template <class T> __device__ __forceinline__ void load8(const T* p, float* o);
template <> __device__ __forceinline__ void load8<float>(const float* p, float* o) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* o) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <class T> __device__ __forceinline__ void store8(T* p, const float* v);
template <> __device__ __forceinline__ void store8<float>(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <> __device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float* v) {
  uint4 o;
  o.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  o.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  o.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
  o.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = o;
}

// Per-row sums in a fixed order.  Thread t owns the 8-element vector t of the
// row (head t / (hd/8)); per-head partials are reduced over the hd/8 threads of
// the head with xor shuffles, then across heads in head order by one thread.
struct RowSums {
  float d, nrm, cks;
};

template <int VPH>  // vectors per head = hd / 8 (8 or 16)
__device__ __forceinline__ float head_reduce(float v) {
#pragma unroll
  for (int o = VPH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// shared scratch: [Hkv][4] partials (diff^2, reuse^2, rec.reuse, rec^2)
template <int VPH>
__device__ RowSums row_sums(const float* a, const float* b, bool active, int Hkv, float* sh) {
  float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
  if (active) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float df = a[i] - b[i];
      p0 += df * df;
      p1 += b[i] * b[i];
      p2 += a[i] * b[i];
      p3 += a[i] * a[i];
    }
  }
  p0 = head_reduce<VPH>(p0);
  p1 = head_reduce<VPH>(p1);
  p2 = head_reduce<VPH>(p2);
  p3 = head_reduce<VPH>(p3);
  const int t = threadIdx.x;
  if (active && (t % VPH) == 0) {
    const int h = t / VPH;
    sh[h * 4 + 0] = p0;
    sh[h * 4 + 1] = p1;
    sh[h * 4 + 2] = p2;
    sh[h * 4 + 3] = p3;
  }
  __syncthreads();
  RowSums s{0.f, 0.f, 0.f};
  for (int h = 0; h < Hkv; h++) {
    s.d += sh[h * 4 + 0];
    s.nrm += sh[h * 4 + 1];
    const float na = sh[h * 4 + 3], nb = sh[h * 4 + 1];
    float c;
    if (na == 0.f && nb == 0.f) c = 1.f;
    else if (na == 0.f || nb == 0.f) c = 0.f;
    else c = sh[h * 4 + 2] / (sqrtf(na) * sqrtf(nb));
    s.cks += c;
  }
  s.cks /= (float)Hkv;
  return s;
}



// ------------------------------------------------------------------ fusion + scatter
// One block per row; thread t owns elements 8t..8t+7 of the [Hkv*hd] row.

template <class T, int VPH>
__global__ void blend_scatter_kernel(int T_max, const int32_t* __restrict__ n_rows,
                                     const int32_t* __restrict__ row_tok, const T* __restrict__ k_rec,
                                     const T* __restrict__ v_rec, T* __restrict__ k_pool, T* __restrict__ v_pool,
                                     int n_slots, const int32_t* __restrict__ src_slot,
                                     const int32_t* __restrict__ dst_slot, int alpha_mode, float* __restrict__ alpha,
                                     float* __restrict__ d_out, float* __restrict__ cksim_out, int Hkv, int hd) {
  __shared__ float sh[4 * 64];
  const int r = blockIdx.x;
  if (r >= row_count(n_rows, T_max)) return;
  const int g = row_tok ? row_tok[r] : r;
  const int dst = dst_slot[r];
  const int t = threadIdx.x;
  const int nvec = Hkv * hd / 8;
  const bool active = t < nvec;
  const int h = t / VPH, e0 = (t % VPH) * 8;
  float kr[8], vr[8], ku[8], vu[8];
  if (active) {
    load8<T>(k_rec + (size_t)r * Hkv * hd + t * 8, kr);
    load8<T>(v_rec + (size_t)r * Hkv * hd + t * 8, vr);
  }
  const int src = src_slot ? src_slot[g] : -1;
  const bool have_src = src_slot && src >= 0 && src < n_slots;
  float a_use = 1.f;
  if (src_slot) {
    if (active) {
      if (have_src) {
        load8<T>(k_pool + pool_off(src, h, Hkv, hd) + e0, ku);
        load8<T>(v_pool + pool_off(src, h, Hkv, hd) + e0, vu);
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++) ku[i] = vu[i] = 0.f;
      }
    }
    const RowSums s = row_sums<VPH>(kr, ku, active, Hkv, sh);
    const float a_new = alpha_rule(s.d, s.nrm);
    if (alpha_mode == KVB_ALPHA_LAG) a_use = alpha ? alpha[g] : 1.f;
    else if (alpha_mode == KVB_ALPHA_CURRENT) a_use = a_new;
    __syncthreads();  // every thread has read alpha[g] before it is overwritten
    if (t == 0) {
      if (alpha && alpha_mode != KVB_ALPHA_ONE) alpha[g] = a_new;
      if (d_out) d_out[r] = s.d;
      if (cksim_out) cksim_out[r] = s.cks;
    }
  }
  if (!active || dst < 0 || dst >= n_slots) return;
  float ko[8], vo[8];
  if (src_slot && a_use != 1.f) {
    const float b = 1.f - a_use;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      ko[i] = a_use * kr[i] + b * ku[i];
      vo[i] = a_use * vr[i] + b * vu[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      ko[i] = kr[i];
      vo[i] = vr[i];
    }
  }
  store8<T>(k_pool + pool_off(dst, h, Hkv, hd) + e0, ko);
  store8<T>(v_pool + pool_off(dst, h, Hkv, hd) + e0, vo);
}

// ------------------------------------------------------------------ RoPE + fusion + scatter
// What rope_kernel followed by blend_scatter_kernel computes, in one pass over
// the row: one block per row.  The Q vectors (8 elements each) are rotated in
// place; then thread t owns vector t of the row's [K | V] (a head's hd / 8
// vectors in consecutive lanes, as in blend_scatter_kernel): K is rotated and
// stored, and K and V are fused with the cached rows and scattered to the new
// slot.  RoPE takes the partner half of each pair from the lane hd / 16 away;
// the per-head K sums use row_sums' butterfly and head order.

// in-place rotate-half of one 8-element vector, vector vi of its head (VPH
// vectors per head): pairs j .. j + 7 with j = (vi % (VPH / 2)) * 8
template <int VPH>
__device__ __forceinline__ void rotate8(float (&x)[8], int vi, const float2* cs) {
  float w[8];
#pragma unroll
  for (int e = 0; e < 8; e++) w[e] = __shfl_xor(x[e], VPH / 2, 64);
  const int j = (vi % (VPH / 2)) * 8;
  if (vi < VPH / 2) {
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = rot_lo(x[e], w[e], cs[j + e].x, cs[j + e].y);
  } else {
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = rot_hi(x[e], w[e], cs[j + e].x, cs[j + e].y);
  }
}

template <class T> __device__ __forceinline__ float round_to(float v);
template <> __device__ __forceinline__ float round_to<float>(float v) { return v; }
template <> __device__ __forceinline__ float round_to<bf16_t>(float v) { return bf2f(f2bf(v)); }

template <class T, int VPH, int QI>
__global__ void __launch_bounds__(1024) rope_fuse_kernel(int T_max, const int32_t* __restrict__ n_rows,
                                                         const int32_t* __restrict__ row_tok,
                                                         const int32_t* __restrict__ tok_pos, T* __restrict__ q,
                                                         T* __restrict__ k, const T* __restrict__ v,
                                                         T* __restrict__ k_pool, T* __restrict__ v_pool, int n_slots,
                                                         const int32_t* __restrict__ src_slot,
                                                         const int32_t* __restrict__ dst_slot, int alpha_mode,
                                                         float* __restrict__ alpha, float* __restrict__ d_out,
                                                         float* __restrict__ cksim_out, int Hq, int Hkv, int hd,
                                                         RopeFreq rf) {
  __shared__ float2 cs[64];
  __shared__ float sh[4 * 64];
  const int r = blockIdx.x;
  if (r >= row_count(n_rows, T_max)) return;
  const int t = threadIdx.x, nth = blockDim.x;
  const int nq = Hq * VPH, nk = Hkv * VPH;
  // every load that depends on the row alone is issued first, so their
  // latencies overlap the token lookups and the angles
  const bool act = t < 2 * nk, is_k = t < nk;
  const int u = is_k ? t : t - nk, h = u / VPH, e0 = (u % VPH) * 8;
  float xq[QI][8], x[8], ru[8];
  T* qr = q + (size_t)r * Hq * hd;
  if (tok_pos) {
#pragma unroll
    for (int i = 0; i < QI; i++) {
      const int iv = i * nth + t;
      if (iv < nq) load8<T>(qr + iv * 8, xq[i]);
      else {
#pragma unroll
        for (int e = 0; e < 8; e++) xq[i][e] = 0.f;
      }
    }
  }
  if (act) load8<T>(is_k ? k + (size_t)r * nk * 8 + u * 8 : v + (size_t)r * nk * 8 + u * 8, x);
  else {
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = 0.f;
  }
  const int g = row_tok ? row_tok[r] : r;
  const int dst = dst_slot[r];  // read now: after the barriers its latency would end the block
  const int src = src_slot ? src_slot[g] : -1;
  const bool have_src = src_slot && src >= 0 && src < n_slots;
#pragma unroll
  for (int e = 0; e < 8; e++) ru[e] = 0.f;
  if (act && have_src) load8<T>((is_k ? k_pool : v_pool) + pool_off(src, h, Hkv, hd) + e0, ru);
  const float a_old = (src_slot && alpha && alpha_mode == KVB_ALPHA_LAG) ? alpha[g] : 1.f;
  if (tok_pos && t < hd / 2) cs[t] = rope_cs(tok_pos[g], rf.f[t]);
  __syncthreads();
  if (tok_pos) {
    // Q rotated in place (every lane runs each step, so the exchanges see whole heads)
#pragma unroll
    for (int i = 0; i < QI; i++) {
      const int iv = i * nth + t;
      rotate8<VPH>(xq[i], iv % VPH, cs);
      if (iv < nq) store8<T>(qr + iv * 8, xq[i]);
    }
    // K rotated and stored; V lanes take part in the exchange and keep their values
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; e++) y[e] = x[e];
    rotate8<VPH>(y, u % VPH, cs);
    if (is_k) {
#pragma unroll
      for (int e = 0; e < 8; e++) x[e] = round_to<T>(y[e]);  // the stored rotated key
      if (act) store8<T>(k + (size_t)r * nk * 8 + u * 8, x);
    }
  }
  float a_use = 1.f;
  if (src_slot) {
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
    if (act && is_k) {
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float df = x[i] - ru[i];
        p0 += df * df;
        p1 += ru[i] * ru[i];
        p2 += x[i] * ru[i];
        p3 += x[i] * x[i];
      }
    }
    p0 = head_reduce<VPH>(p0);
    p1 = head_reduce<VPH>(p1);
    p2 = head_reduce<VPH>(p2);
    p3 = head_reduce<VPH>(p3);
    if (act && is_k && (u % VPH) == 0) {
      sh[h * 4 + 0] = p0;
      sh[h * 4 + 1] = p1;
      sh[h * 4 + 2] = p2;
      sh[h * 4 + 3] = p3;
    }
    __syncthreads();
    float d = 0.f, nrm = 0.f, cks = 0.f;
    for (int hh = 0; hh < Hkv; hh++) {
      d += sh[hh * 4 + 0];
      nrm += sh[hh * 4 + 1];
      const float na = sh[hh * 4 + 3], nb = sh[hh * 4 + 1];
      float c;
      if (na == 0.f && nb == 0.f) c = 1.f;
      else if (na == 0.f || nb == 0.f) c = 0.f;
      else c = sh[hh * 4 + 2] / (sqrtf(na) * sqrtf(nb));
      cks += c;
    }
    cks /= (float)Hkv;
    const float a_new = alpha_rule(d, nrm);
    if (alpha_mode == KVB_ALPHA_LAG) a_use = a_old;
    else if (alpha_mode == KVB_ALPHA_CURRENT) a_use = a_new;
    // alpha[g] was read before the first barrier, so thread 0 may overwrite it
    if (t == 0) {
      if (alpha && alpha_mode != KVB_ALPHA_ONE) alpha[g] = a_new;
      if (d_out) d_out[r] = d;
      if (cksim_out) cksim_out[r] = cks;
    }
  }
  if (!act || dst < 0 || dst >= n_slots) return;
  float o[8];
  if (src_slot && a_use != 1.f) {
    const float b = 1.f - a_use;
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] = a_use * x[i] + b * ru[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] = x[i];
  }
  store8<T>((is_k ? k_pool : v_pool) + pool_off(dst, h, Hkv, hd) + e0, o);
}

// ------------------------------------------------------------------ deviation (layer 1)
// d[g], alpha[g] and the 64-bit sort key (~bits(d) << 32 | g) for every token.

template <class T, int VPH>
__global__ void deviation_kernel(int n_tok, const T* __restrict__ k_rec, const T* __restrict__ k_pool, int n_slots,
                                 const int32_t* __restrict__ reuse_slot, float* __restrict__ d,
                                 float* __restrict__ alpha, int Hkv, int hd) {
  __shared__ float sh[4 * 64];
  const int g = blockIdx.x;
  if (g >= n_tok) return;
  const int t = threadIdx.x;
  const int nvec = Hkv * hd / 8;
  const bool active = t < nvec;
  const int h = t / VPH, e0 = (t % VPH) * 8;
  float kr[8], ku[8];
  const int src = reuse_slot[g];
  const bool have = src >= 0 && src < n_slots;
  if (active) {
    load8<T>(k_rec + (size_t)g * Hkv * hd + t * 8, kr);
    if (have) load8<T>(k_pool + pool_off(src, h, Hkv, hd) + e0, ku);
    else {
#pragma unroll
      for (int i = 0; i < 8; i++) ku[i] = 0.f;
    }
  }
  const RowSums s = row_sums<VPH>(kr, ku, active, Hkv, sh);
  if (t == 0) {
    d[g] = s.d;
    alpha[g] = alpha_rule(s.d, s.nrm);
  }
}

__device__ __forceinline__ void unpack8_bf16(const uint4& a, float (&f)[8]) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// The same d and alpha, bitwise (per-vector sums of 8 elements, the butterfly
// over a head's lanes and the sum over heads in head order, as in row_sums),
// with one wave per DEV_TPW tokens: every slot, K and cached-K load of the
// wave's tokens is issued before any is used, so more bytes are in flight
// than with one block and its LDS reduction per token.  (bf16, Hkv * hd a
// multiple of 512.)
constexpr int DEV_TPW = 4;
template <int VPH, int NV>
__global__ void __launch_bounds__(256) deviation_wave_kernel(int n_tok, const bf16_t* __restrict__ k_rec,
                                                             const bf16_t* __restrict__ k_pool, int n_slots,
                                                             const int32_t* __restrict__ reuse_slot,
                                                             float* __restrict__ d, float* __restrict__ alpha, int Hkv,
                                                             int hd) {
  constexpr int HPV = 64 / VPH;  // heads per 64 vectors
  const int lane = threadIdx.x & 63;
  const int g0 = (blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * DEV_TPW;
  if (g0 >= n_tok) return;
  int sl = -1;
  if (lane < DEV_TPW && g0 + lane < n_tok) sl = reuse_slot[g0 + lane];
  uint4 ar[DEV_TPW][NV], br[DEV_TPW][NV];
#pragma unroll
  for (int i = 0; i < DEV_TPW; i++) {
    const int src = __builtin_amdgcn_readlane(sl, i);
    const bool in = g0 + i < n_tok;
    const bool have = in && src >= 0 && src < n_slots;
#pragma unroll
    for (int v = 0; v < NV; v++) {
      const int t = lane + 64 * v, h = t / VPH, e0 = (t % VPH) * 8;
      ar[i][v] = in ? *reinterpret_cast<const uint4*>(k_rec + (size_t)(g0 + i) * Hkv * hd + t * 8)
                    : make_uint4(0, 0, 0, 0);
      br[i][v] = have ? *reinterpret_cast<const uint4*>(k_pool + pool_off(src, h, Hkv, hd) + e0)
                      : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < DEV_TPW; i++) {
    if (g0 + i >= n_tok) break;
    float p0[NV], p1[NV];
#pragma unroll
    for (int v = 0; v < NV; v++) {
      float a[8], b[8];
      unpack8_bf16(ar[i][v], a);
      unpack8_bf16(br[i][v], b);
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float df = a[e] - b[e];
        s0 += df * df;
        s1 += b[e] * b[e];
      }
      p0[v] = head_reduce<VPH>(s0);
      p1[v] = head_reduce<VPH>(s1);
    }
    float sd = 0.f, sn = 0.f;
#pragma unroll
    for (int v = 0; v < NV; v++)
#pragma unroll
      for (int hh = 0; hh < HPV; hh++) {
        sd += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p0[v]), hh * VPH));
        sn += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p1[v]), hh * VPH));
      }
    if (lane == 0) {
      d[g0 + i] = sd;
      alpha[g0 + i] = alpha_rule(sd, sn);
    }
  }
}

template <class T>
kvb_status launch_deviation(hipStream_t st, int n_tok, const void* k_rec, const void* k_pool, int n_pages,
                            const int32_t* reuse_slot, float* d, float* alpha, int Hkv, int hd) {
  const int nvec = Hkv * hd / 8;
  const int threads = ((nvec + 63) / 64) * 64;
  if (n_tok == 0) return KVB_OK;
  LaunchTimer lt(st, "deviation");
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int nv = nvec / 64;
    if (nvec % 64 == 0 && (nv == 1 || nv == 2 || nv == 4)) {
      const dim3 grid(cdiv(n_tok, 4 * DEV_TPW)), block(256);
      const bf16_t* kr = (const bf16_t*)k_rec;
      const bf16_t* kp = (const bf16_t*)k_pool;
      const int ns = n_pages * 16;
      if (hd == 128) {
        if (nv == 1) deviation_wave_kernel<16, 1><<<grid, block, 0, st>>>(n_tok, kr, kp, ns, reuse_slot, d, alpha, Hkv, hd);
        else if (nv == 2) deviation_wave_kernel<16, 2><<<grid, block, 0, st>>>(n_tok, kr, kp, ns, reuse_slot, d, alpha, Hkv, hd);
        else deviation_wave_kernel<16, 4><<<grid, block, 0, st>>>(n_tok, kr, kp, ns, reuse_slot, d, alpha, Hkv, hd);
      } else {
        if (nv == 1) deviation_wave_kernel<8, 1><<<grid, block, 0, st>>>(n_tok, kr, kp, ns, reuse_slot, d, alpha, Hkv, hd);
        else if (nv == 2) deviation_wave_kernel<8, 2><<<grid, block, 0, st>>>(n_tok, kr, kp, ns, reuse_slot, d, alpha, Hkv, hd);
        else deviation_wave_kernel<8, 4><<<grid, block, 0, st>>>(n_tok, kr, kp, ns, reuse_slot, d, alpha, Hkv, hd);
      }
      return check_launch("deviation_wave_kernel");
    }
  }
  if (hd == 128)
    deviation_kernel<T, 16><<<n_tok, threads, 0, st>>>(n_tok, (const T*)k_rec, (const T*)k_pool, n_pages * 16,
                                                        reuse_slot, d, alpha, Hkv, hd);
  else
    deviation_kernel<T, 8><<<n_tok, threads, 0, st>>>(n_tok, (const T*)k_rec, (const T*)k_pool, n_pages * 16,
                                                       reuse_slot, d, alpha, Hkv, hd);
  return check_launch("deviation_kernel");
}
template kvb_status launch_deviation<float>(hipStream_t, int, const void*, const void*, int, const int32_t*, float*,
                                            float*, int, int);
template kvb_status launch_deviation<bf16_t>(hipStream_t, int, const void*, const void*, int, const int32_t*, float*,
                                             float*, int, int);

template <class T>
kvb_status launch_rope(hipStream_t st, int T_max, const int32_t* n_rows, const int32_t* row_tok,
                       const int32_t* tok_pos, void* q, void* k, const kvb_model_desc* d) {
  if (T_max == 0) return KVB_OK;
  LaunchTimer lt(st, "rope");
  rope_kernel<T><<<T_max, 256, 0, st>>>(T_max, n_rows, row_tok, tok_pos, (T*)q, (T*)k, d->n_q_heads, d->n_kv_heads,
                                        d->head_dim, rope_freq(d->head_dim, d->rope_base));
  return check_launch("rope_kernel");
}
template kvb_status launch_rope<float>(hipStream_t, int, const int32_t*, const int32_t*, const int32_t*, void*, void*,
                                       const kvb_model_desc*);
template kvb_status launch_rope<bf16_t>(hipStream_t, int, const int32_t*, const int32_t*, const int32_t*, void*, void*,
                                        const kvb_model_desc*);

// ------------------------------------------------------------------ slot maps

__global__ void copy_slots_kernel(int n_tok, const int32_t* __restrict__ reuse_slot, int32_t* __restrict__ slot_map) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g < n_tok) slot_map[g] = reuse_slot ? reuse_slot[g] : -1;
}

__global__ void scatter_slots_kernel(int B, int T_max, const int32_t* __restrict__ cu_rows,
                                     const int32_t* __restrict__ row_tok, const int32_t* __restrict__ new_pages,
                                     const int32_t* __restrict__ cu_pages, int32_t* __restrict__ slot_map,
                                     int32_t* __restrict__ dst_slot, int n_tok, int n_pages,
                                     int32_t* __restrict__ page_dirty) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= T_max || r >= cu_rows[B]) return;
  int lo = 0, hi = B;  // find b with cu_rows[b] <= r < cu_rows[b+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_rows[mid] <= r) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int j = r - cu_rows[b];
  const int np = cu_pages[b + 1] - cu_pages[b];
  int slot = -1;
  if ((j >> 4) < np) slot = new_pages[cu_pages[b] + (j >> 4)] * 16 + (j & 15);
  if (dst_slot) dst_slot[r] = slot;
  const int g = row_tok ? row_tok[r] : r;
  if (slot >= 0 && g >= 0 && g < n_tok) slot_map[g] = slot;
  // SLIDE's dirty-page counter: one more selected token routed into this page
  if (page_dirty && slot >= 0 && (slot >> 4) < n_pages) atomicAdd(&page_dirty[slot >> 4], 1);
}

// page_dirty[slot / 16] += 1 for every valid slot of rows r < *n_rows
__global__ void page_dirty_add_kernel(int T_max, const int32_t* __restrict__ n_rows, const int32_t* __restrict__ slots,
                                      int n_pages, int32_t* __restrict__ page_dirty) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= T_max || (n_rows && r >= *n_rows)) return;
  const int s = slots[r];
  if (s >= 0 && (s >> 4) < n_pages) atomicAdd(&page_dirty[s >> 4], 1);
}

}  // namespace kvb

using namespace kvb;

// ------------------------------------------------------------------ entry points

extern "C" kvb_status kvb_embed(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                                const int32_t* n_rows, const int32_t* row_tok, const int32_t* tokens, int32_t vocab,
                                const void* table, void* hidden) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0 || vocab <= 0) return fail(KVB_ERR_INVALID_ARG, "T_max < 0 or vocab <= 0");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(tokens, "tokens");
  KVB_CHECK_PTR(table, "table");
  KVB_CHECK_PTR(hidden, "hidden");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  LaunchTimer lt(st, "embed");
  if (desc->dtype == KVB_BF16)
    embed_kernel<bf16_t><<<T_max, 256, 0, st>>>(T_max, n_rows, row_tok, tokens, vocab, (const bf16_t*)table,
                                                (bf16_t*)hidden, desc->d_model);
  else
    embed_kernel<float><<<T_max, 256, 0, st>>>(T_max, n_rows, row_tok, tokens, vocab, (const float*)table,
                                               (float*)hidden, desc->d_model);
  return check_launch("embed_kernel");
}

extern "C" kvb_status kvb_rope(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                               const int32_t* n_rows, const int32_t* row_tok, const int32_t* tok_pos, void* q,
                               void* k) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0) return fail(KVB_ERR_INVALID_ARG, "T_max < 0");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(tok_pos, "tok_pos");
  KVB_CHECK_PTR(q, "q");
  KVB_CHECK_PTR(k, "k");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  if (desc->dtype == KVB_BF16) return launch_rope<bf16_t>(st, T_max, n_rows, row_tok, tok_pos, q, k, desc);
  return launch_rope<float>(st, T_max, n_rows, row_tok, tok_pos, q, k, desc);
}

extern "C" kvb_status kvb_blend_scatter(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                                        const int32_t* n_rows, const int32_t* row_tok, const void* k_rec,
                                        const void* v_rec, void* k_pool, void* v_pool, int32_t n_pages,
                                        const int32_t* src_slot, const int32_t* dst_slot, int32_t alpha_mode,
                                        float* alpha, float* d_out, float* cksim_out) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0 || n_pages < 0) return fail(KVB_ERR_INVALID_ARG, "T_max or n_pages < 0");
  if (alpha_mode < KVB_ALPHA_LAG || alpha_mode > KVB_ALPHA_ONE) return fail(KVB_ERR_INVALID_ARG, "bad alpha_mode");
  if (!src_slot && (alpha_mode != KVB_ALPHA_ONE || d_out || cksim_out))
    return fail(KVB_ERR_INVALID_ARG, "without src_slot only KVB_ALPHA_ONE with no d_out/cksim_out is allowed");
  if (alpha_mode == KVB_ALPHA_LAG && !alpha) return fail(KVB_ERR_INVALID_ARG, "KVB_ALPHA_LAG needs alpha");
  if ((long)n_pages * 16 > 0x7fffffffL) return fail(KVB_ERR_INVALID_ARG, "too many pages for int32 slots");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(k_rec, "k_rec");
  KVB_CHECK_PTR(v_rec, "v_rec");
  KVB_CHECK_PTR(k_pool, "k_pool");
  KVB_CHECK_PTR(v_pool, "v_pool");
  KVB_CHECK_PTR(dst_slot, "dst_slot");
  const int Hkv = desc->n_kv_heads, hd = desc->head_dim;
  const int nvec = Hkv * hd / 8;
  if (nvec > 1024 || Hkv > 64) return fail(KVB_ERR_UNSUPPORTED, "n_kv_heads * head_dim must be <= 8192");
  const int threads = ((nvec + 63) / 64) * 64;
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  const int ns = n_pages * 16;
  LaunchTimer lt(st, "blend_scatter");
#define KVB_BLEND(T, VPH)                                                                                   \
  blend_scatter_kernel<T, VPH><<<T_max, threads, 0, st>>>(T_max, n_rows, row_tok, (const T*)k_rec,         \
                                                          (const T*)v_rec, (T*)k_pool, (T*)v_pool, ns, src_slot, \
                                                          dst_slot, alpha_mode, alpha, d_out, cksim_out, Hkv, hd)
  if (desc->dtype == KVB_BF16) {
    if (hd == 128) KVB_BLEND(bf16_t, 16);
    else KVB_BLEND(bf16_t, 8);
  } else {
    if (hd == 128) KVB_BLEND(float, 16);
    else KVB_BLEND(float, 8);
  }
#undef KVB_BLEND
  return check_launch("blend_scatter_kernel");
}

extern "C" kvb_status kvb_slot_map(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t B, int32_t n_tok,
                                   int32_t T_max, const int32_t* cu_rows, const int32_t* row_tok,
                                   const int32_t* reuse_slot, const int32_t* new_pages, const int32_t* cu_pages,
                                   int32_t* slot_map, int32_t* dst_slot, int32_t n_pages, int32_t* page_dirty) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (B < 0 || n_tok < 0 || T_max < 0 || n_pages < 0) return fail(KVB_ERR_INVALID_ARG, "negative size");
  KVB_CHECK_PTR(slot_map, "slot_map");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  if (n_tok > 0) {
    LaunchTimer lt(st, "slot_copy");
    copy_slots_kernel<<<cdiv(n_tok, 256), 256, 0, st>>>(n_tok, reuse_slot, slot_map);
    KVB_TRY(check_launch("copy_slots_kernel"));
  }
  if (B == 0 || T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(cu_rows, "cu_rows");
  KVB_CHECK_PTR(new_pages, "new_pages");
  KVB_CHECK_PTR(cu_pages, "cu_pages");
  LaunchTimer lt(st, "slot_scatter");
  scatter_slots_kernel<<<cdiv(T_max, 256), 256, 0, st>>>(B, T_max, cu_rows, row_tok, new_pages, cu_pages, slot_map,
                                                         dst_slot, n_tok, n_pages, page_dirty);
  return check_launch("scatter_slots_kernel");
}

extern "C" kvb_status kvb_page_dirty_add(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                                         const int32_t* n_rows, const int32_t* slots, int32_t n_pages,
                                         int32_t* page_dirty) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0 || n_pages < 0) return fail(KVB_ERR_INVALID_ARG, "negative size");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(slots, "slots");
  KVB_CHECK_PTR(page_dirty, "page_dirty");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  LaunchTimer lt(st, "page_dirty");
  page_dirty_add_kernel<<<cdiv(T_max, 256), 256, 0, st>>>(T_max, n_rows, slots, n_pages, page_dirty);
  return check_launch("page_dirty_add_kernel");
}

extern "C" kvb_status kvb_qkv_fused(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                                    const int32_t* n_rows, const int32_t* row_tok, const void* hidden,
                                    const void* norm_w, const void* w_qkv, const int32_t* tok_pos, void* q, void* k,
                                    void* v, void* k_pool, void* v_pool, int32_t n_pages, const int32_t* src_slot,
                                    const int32_t* dst_slot, int32_t alpha_mode, float* alpha, float* d_out,
                                    float* cksim_out, void* ws, size_t ws_bytes, int32_t flags) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0 || n_pages < 0) return fail(KVB_ERR_INVALID_ARG, "negative size");
  if (alpha_mode != KVB_ALPHA_LAG && alpha_mode != KVB_ALPHA_CURRENT && alpha_mode != KVB_ALPHA_ONE)
    return fail(KVB_ERR_INVALID_ARG, "bad alpha_mode");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(k_pool, "k_pool");
  KVB_CHECK_PTR(v_pool, "v_pool");
  KVB_CHECK_PTR(dst_slot, "dst_slot");
  if (!src_slot && (alpha_mode != KVB_ALPHA_ONE || d_out || cksim_out))
    return fail(KVB_ERR_INVALID_ARG, "without src_slot only KVB_ALPHA_ONE and no d_out / cksim_out");
  if ((long)n_pages * 16 > 0x7fffffffL) return fail(KVB_ERR_INVALID_ARG, "too many pages for int32 slots");
  const int Hkv = desc->n_kv_heads, hd = desc->head_dim;
  if (desc->dtype == KVB_BF16 && T_max == 1 && flags == KVB_QKV_SPLIT_K && !src_slot && tok_pos &&
      desc->d_model % 8 == 0 && desc->d_model <= 32768) {
    // one row replacing nothing cached (decode): RoPE and the K/V store run in
    // the epilogue of the one-row product, no separate pass
    KVB_CHECK_PTR(hidden, "hidden");
    KVB_CHECK_PTR(w_qkv, "w_qkv");
    KVB_CHECK_PTR(q, "q");
    KVB_CHECK_PTR(k, "k");
    KVB_CHECK_PTR(v, "v");
    const size_t need = ws_qkv_bytes(desc, T_max) + ws_gemm_sk_bytes(0);
    if (!ws || ws_bytes < need) return fail(KVB_ERR_WORKSPACE, "kvb_qkv_fused workspace too small");
    CtxScope scope(ctx);
    return qkv_rope_one_row((hipStream_t)stream, desc, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v,
                            k_pool, v_pool, n_pages * 16, dst_slot, ws);
  }
  const int nkv = 2 * Hkv * hd / 8;  // K and V vectors of a row, one per thread
  if (nkv > 1024 || Hkv > 64 || (long)desc->n_q_heads * hd / 8 > 8L * std::max(64, (nkv + 63) / 64 * 64)) {
    KVB_TRY(kvb_qkv_proj(ctx, stream, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v, ws,
                         ws_bytes, flags));
    return kvb_blend_scatter(ctx, stream, desc, T_max, n_rows, row_tok, k, v, k_pool, v_pool, n_pages, src_slot,
                             dst_slot, alpha_mode, alpha, d_out, cksim_out);
  }
  // the projection without RoPE, then the rotation, fusion and scatter in one pass
  KVB_TRY(kvb_qkv_proj(ctx, stream, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, nullptr, q, k, v, ws,
                       ws_bytes, flags));
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  const int threads = std::max(64, (nkv + 63) / 64 * 64);
  const int qi = cdiv((long)desc->n_q_heads * hd / 8, threads);  // Q vectors per thread
  const RopeFreq rf = rope_freq(hd, desc->rope_base);
  const int ns = n_pages * 16;
  LaunchTimer lt(st, "rope_fuse");
#define KVB_ROPE_FUSE(T, VPH, QI)                                                                              \
  rope_fuse_kernel<T, VPH, QI><<<T_max, threads, 0, st>>>(T_max, n_rows, row_tok, tok_pos, (T*)q, (T*)k,       \
                                                          (const T*)v, (T*)k_pool, (T*)v_pool, ns, src_slot,   \
                                                          dst_slot, alpha_mode, alpha, d_out, cksim_out,       \
                                                          desc->n_q_heads, Hkv, hd, rf)
#define KVB_ROPE_FUSE_QI(T, VPH)                     \
  if (qi <= 1) KVB_ROPE_FUSE(T, VPH, 1);             \
  else if (qi <= 2) KVB_ROPE_FUSE(T, VPH, 2);        \
  else if (qi <= 4) KVB_ROPE_FUSE(T, VPH, 4);        \
  else KVB_ROPE_FUSE(T, VPH, 8);
  if (desc->dtype == KVB_BF16) {
    if (hd == 128) { KVB_ROPE_FUSE_QI(bf16_t, 16) }
    else { KVB_ROPE_FUSE_QI(bf16_t, 8) }
  } else {
    if (hd == 128) { KVB_ROPE_FUSE_QI(float, 16) }
    else { KVB_ROPE_FUSE_QI(float, 8) }
  }
#undef KVB_ROPE_FUSE_QI
#undef KVB_ROPE_FUSE
  return check_launch("rope_fuse_kernel");
}
