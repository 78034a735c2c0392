// Sparse-query causal attention over the paged, spliced KV of one layer
// (EPIC page, section 4, LegoLink steps 3-5: Q of the k' recomputed rows
// against K_exp / V_exp of all N tokens, causal mask, softmax, times V).
//
// bf16 path (gfx950 MFMA, flash-style online softmax):
//   * one block = one KV head x 256 query rows, a query row being a (token,
//     query head of the GQA group) pair, so the whole group shares every K/V
//     tile; 4 waves x 64 query rows (two 32-wide MFMA column tiles);
//   * key tiles of 64 tokens are gathered row by row through the per-token
//     slot map, prefetched into registers while the previous tile computes;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane ends with 16 scores of
//     one query, which is already the B-operand layout of O^T = V^T P^T, so
//     probabilities stay in registers; softmax statistics need one xor-32
//     exchange per query;
//   * the V tile is stored transposed (dims x keys) with key bits 2 and 3
//     swapped, so each V^T operand is one 16-byte LDS read;
//   * only tiles that cross a query's causal edge or its lower bound are
//     masked; blocks run longest first;
//   * split-KV: with few query blocks the key range of each block is cut into
//     n_split parts whose partial (O, max, sum) a merge kernel combines.
// fp32 path: one wave per (row, query head), plain online softmax.
#include "common.h"

namespace kvb {

__device__ __forceinline__ size_t kv_off(int slot, int h, int Hkv, int hd) {
  return (((size_t)(slot >> 4) * Hkv + h) * 16 + (slot & 15)) * hd;
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, b2_t));
}

constexpr int AQ = 256;        // query rows per block
constexpr int AKT = 64;        // keys per tile
constexpr int ATHREADS = 256;

struct AttnArgs {
  int T_max;
  const int32_t* n_rows;
  const int32_t* row_tok;
  const int32_t* tok_lo;
  const bf16_t* q;
  const bf16_t* k_pool;
  const bf16_t* v_pool;
  int n_slots;
  const int32_t* slot_map;
  float scale_log2;
  bf16_t* o;
  int Hq, Hkv;
  int n_qblocks, n_split;
  float* part_o;   // [n_split][T_max][Hq][HD] (n_split > 1)
  float* part_ml;  // [n_split][T_max][Hq][2]
};

template <int HD>
__global__ void __launch_bounds__(ATHREADS) attn_bf16_kernel(AttnArgs a) {
  constexpr int LDK_ = HD + 8;     // K tile row stride (bf16)
  constexpr int LDV_ = AKT + 8;    // transposed V tile row stride (bf16)
  constexpr int KS = HD / 16;      // k16 steps of Q K^T
  constexpr int DT = HD / 32;      // 32-wide dim tiles of P V
  constexpr int CPR = HD / 8;      // 16-byte chunks per K/V row
  constexpr int LOADS = AKT * CPR / ATHREADS;
  __shared__ __align__(16) bf16_t sK[AKT * LDK_];
  __shared__ __align__(16) bf16_t sVt[HD * LDV_];
  __shared__ int s_kmin, s_kmax, s_pmin, s_lomax;

  const int G = a.Hq / a.Hkv;
  const int TB = AQ / G;  // tokens per block
  const int M = row_count(a.n_rows, a.T_max);
  const int qb = a.n_qblocks - 1 - (int)blockIdx.x;  // longest first
  const int h = blockIdx.y, split = blockIdx.z;
  const int r0 = qb * TB;
  if (r0 >= M) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, g2 = lane >> 5;

  if (t == 0) {
    s_kmin = 0x7fffffff;
    s_kmax = -1;
    s_pmin = 0x7fffffff;
    s_lomax = -1;
  }
  __syncthreads();
  if (t < TB && r0 + t < M) {
    const int g = a.row_tok ? a.row_tok[r0 + t] : r0 + t;
    const int lo = a.tok_lo[g];
    atomicMin(&s_kmin, lo);
    atomicMax(&s_kmax, g);
    atomicMin(&s_pmin, g);
    atomicMax(&s_lomax, lo);
  }
  __syncthreads();
  // this split's share of the block's key range, in whole tiles
  const int kmin = s_kmin, kmax = s_kmax, pmin = s_pmin, lomax = s_lomax;
  const int ntiles = (kmax - kmin) / AKT + 1;
  const int t_begin = (int)((long)ntiles * split / a.n_split);
  const int t_end = (int)((long)ntiles * (split + 1) / a.n_split);

  // this lane's queries: column l32 of query tiles qt = 0, 1
  int qpos[2], qlo[2];
  bool qvalid[2];
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    const int m = wave * 64 + qt * 32 + l32;
    const int r = r0 + m / G, hq = h * G + m % G;
    qvalid[qt] = r < M;
    if (qvalid[qt]) {
      const int g = a.row_tok ? a.row_tok[r] : r;
      qpos[qt] = g;
      qlo[qt] = a.tok_lo[g];
      const bf16_t* qp = a.q + ((size_t)r * a.Hq + hq) * HD + g2 * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        qf[qt][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + ks * 16));
    } else {
      qpos[qt] = -1;
      qlo[qt] = 0x7fffffff;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) qf[qt][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
    }
  }

  f32x16_t oacc[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) oacc[dt][0] = oacc[dt][1] = (f32x16_t){};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};

  uint4 rk[LOADS], rv[LOADS];
  // chunk c = t + 256 i: key c / CPR, part c % CPR
#define ATTN_GLOAD(J0)                                                        \
  _Pragma("unroll") for (int i = 0; i < LOADS; i++) {                         \
    const int c = t + ATHREADS * i;                                           \
    const int key = (J0) + c / CPR, part = c % CPR;                           \
    int slot = -1;                                                            \
    if (key <= kmax) slot = a.slot_map[key];                                  \
    if (slot >= 0 && slot < a.n_slots) {                                      \
      const size_t off = kv_off(slot, h, a.Hkv, HD) + part * 8;               \
      rk[i] = *reinterpret_cast<const uint4*>(a.k_pool + off);                \
      rv[i] = *reinterpret_cast<const uint4*>(a.v_pool + off);                \
    } else {                                                                  \
      rk[i] = rv[i] = make_uint4(0, 0, 0, 0);                                 \
    }                                                                         \
  }

  if (t_begin < t_end) {
    ATTN_GLOAD(kmin + t_begin * AKT);
  }
  for (int ti = t_begin; ti < t_end; ti++) {
    const int j0 = kmin + ti * AKT;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = t + ATHREADS * i;
      const int key = c / CPR, part = c % CPR;
      *reinterpret_cast<uint4*>(sK + key * LDK_ + part * 8) = rk[i];
      // key k = 16 c + 8 h + 4 g + r goes to column 16 c + 8 g + 4 h + r (bits 2 and 3 swapped)
      const int col = (key & ~15) | ((key & 4) << 1) | ((key & 8) >> 1) | (key & 3);
      const uint32_t w[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        sVt[(part * 8 + 2 * e) * LDV_ + col] = (bf16_t)(w[e] & 0xffffu);
        sVt[(part * 8 + 2 * e + 1) * LDV_ + col] = (bf16_t)(w[e] >> 16);
      }
    }
    __syncthreads();
    if (ti + 1 < t_end) {
      ATTN_GLOAD(j0 + AKT);
    }
    const bool need_mask = (j0 + AKT - 1 > pmin) || (j0 < lomax);

    // S^T[kt][qt]: keys j0 + 32 kt + 8 (r / 4) + 4 g2 + r % 4, query column l32 of tile qt
    f32x16_t st[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      st[kt][0] = st[kt][1] = (f32x16_t){};
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const bf16x8_t kf = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(sK + (kt * 32 + l32) * LDK_ + ks * 16 + g2 * 8));
        st[kt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[0][ks], st[kt][0], 0, 0, 0);
        st[kt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[1][ks], st[kt][1], 0, 0, 0);
      }
    }
    // online softmax per query (its 64 scores: 32 in this lane, 32 in lane ^ 32)
    uint4 pf[2][4];  // [qt][16-key step c]: bf16 B operand of the PV product
#pragma unroll
    for (int qt = 0; qt < 2; qt++) {
      float sv[32];
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        const f32x16_t x = st[kt][qt];
#pragma unroll
        for (int r = 0; r < 16; r++) sv[kt * 16 + r] = x[r] * a.scale_log2;
      }
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 32; i++) {
          const int key = j0 + (i >> 4) * 32 + 8 * ((i & 15) >> 2) + 4 * g2 + (i & 3);
          if (key > qpos[qt] || key < qlo[qt]) sv[i] = -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 32; i++) mx = fmaxf(mx, sv[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qt], mx);
      const bool dead = mnew == -INFINITY;
      const float corr = dead ? 1.f : exp2f(mrow[qt] - mnew);
      mrow[qt] = mnew;
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 32; i++) {
        sv[i] = dead ? 0.f : exp2f(sv[i] - mnew);
        ls += sv[i];
      }
      lrow[qt] = lrow[qt] * corr + ls;
      {
        // (a splat-vector product: the scalar form trips a backend crash in this toolchain)
        const f32x16_t cv = {corr, corr, corr, corr, corr, corr, corr, corr,
                             corr, corr, corr, corr, corr, corr, corr, corr};
#pragma unroll
        for (int dt = 0; dt < DT; dt++) oacc[dt][qt] = oacc[dt][qt] * cv;
      }
      // k step c covers keys 16 c .. 16 c + 15: tile kt = c / 2, registers r = 8 (c % 2) .. + 7
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const int b = (c >> 1) * 16 + (c & 1) * 8;
        pf[qt][c] = make_uint4(pack2_bf16(sv[b + 0], sv[b + 1]), pack2_bf16(sv[b + 2], sv[b + 3]),
                               pack2_bf16(sv[b + 4], sv[b + 5]), pack2_bf16(sv[b + 6], sv[b + 7]));
      }
    }
    // O^T[dt][qt] += V^T[dims dt*32 .. +31][keys of step c] P^T
#pragma unroll
    for (int c = 0; c < 4; c++) {
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(sVt + (dt * 32 + l32) * LDV_ + 16 * c + 8 * g2));
        oacc[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8_t, pf[0][c]),
                                                               oacc[dt][0], 0, 0, 0);
        oacc[dt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8_t, pf[1][c]),
                                                               oacc[dt][1], 0, 0, 0);
      }
    }
  }
#undef ATTN_GLOAD

  // oacc[dt][qt][r] = O[query l32 of tile qt][dim dt*32 + 8 (r / 4) + 4 g2 + r % 4]
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    float l = lrow[qt];
    l += __shfl_xor(l, 32, 64);
    if (!qvalid[qt]) continue;
    const int m = wave * 64 + qt * 32 + l32;
    const int r = r0 + m / G, hq = h * G + m % G;
    if (a.n_split == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      bf16_t* op = a.o + ((size_t)r * a.Hq + hq) * HD;
#pragma unroll
      for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const f32x16_t x = oacc[dt][qt];
          uint2 w;
          w.x = pack2_bf16(x[q4 * 4 + 0] * inv, x[q4 * 4 + 1] * inv);
          w.y = pack2_bf16(x[q4 * 4 + 2] * inv, x[q4 * 4 + 3] * inv);
          *reinterpret_cast<uint2*>(op + dt * 32 + 8 * q4 + 4 * g2) = w;
        }
    } else {
      const size_t row = ((size_t)split * a.T_max + r) * a.Hq + hq;
      float* op = a.part_o + row * HD;
#pragma unroll
      for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const f32x16_t x = oacc[dt][qt];
          *reinterpret_cast<float4*>(op + dt * 32 + 8 * q4 + 4 * g2) =
              make_float4(x[q4 * 4 + 0], x[q4 * 4 + 1], x[q4 * 4 + 2], x[q4 * 4 + 3]);
        }
      if (g2 == 0) {
        a.part_ml[row * 2 + 0] = mrow[qt];
        a.part_ml[row * 2 + 1] = l;
      }
    }
  }
}

// merge of split-KV partials: one wave per (row, head); base-2 exponents
template <int HD>
__global__ void __launch_bounds__(256) attn_merge_kernel(int T_max, const int32_t* __restrict__ n_rows, int Hq,
                                                         int n_split, const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, bf16_t* __restrict__ o) {
  const int w = (blockIdx.x * blockDim.x + threadIdx.x) >> 6, lane = threadIdx.x & 63;
  const int M = row_count(n_rows, T_max);
  if (w >= M * Hq) return;
  float mx = -INFINITY;
  for (int s = 0; s < n_split; s++) mx = fmaxf(mx, part_ml[((size_t)s * T_max * Hq + w) * 2]);
  float l = 0.f;
  float acc[HD / 64] = {};
  for (int s = 0; s < n_split; s++) {
    const size_t row = (size_t)s * T_max * Hq + w;
    const float ms = part_ml[row * 2], ls = part_ml[row * 2 + 1];
    const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
    l += ls * f;
#pragma unroll
    for (int e = 0; e < HD / 64; e++) acc[e] += f * part_o[row * HD + lane + 64 * e];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < HD / 64; e++)
    o[(size_t)w * HD + lane + 64 * e] = (bf16_t)(pack2_bf16(acc[e] * inv, 0.f) & 0xffffu);
}

// ------------------------------------------------------------------ fp32 kernel
// one wave per (row, query head); keys in chunks of 64, one key per lane

template <int HD>
__global__ void __launch_bounds__(64) attn_f32_kernel(int T_max, const int32_t* __restrict__ n_rows,
                                                      const int32_t* __restrict__ row_tok,
                                                      const int32_t* __restrict__ tok_lo, const float* __restrict__ q,
                                                      const float* __restrict__ k_pool,
                                                      const float* __restrict__ v_pool, int n_slots,
                                                      const int32_t* __restrict__ slot_map, float scale,
                                                      float* __restrict__ o, int Hq, int Hkv) {
  const int r = blockIdx.x, hq = blockIdx.y;
  if (r >= row_count(n_rows, T_max)) return;
  const int lane = threadIdx.x;
  const int g = row_tok ? row_tok[r] : r;
  const int lo = tok_lo[g];
  const int h = hq / (Hq / Hkv);
  __shared__ float sq[HD];
  for (int i = lane; i < HD; i += 64) sq[i] = q[((size_t)r * Hq + hq) * HD + i];
  __syncthreads();
  constexpr int DPL = HD / 64;  // dims per lane
  float acc[DPL] = {};
  float m = -INFINITY, l = 0.f;
  for (int j0 = lo; j0 <= g; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    int slot = -1;
    if (j <= g) {
      slot = slot_map[j];
      if (slot >= 0 && slot < n_slots) {
        const float* kp = k_pool + kv_off(slot, h, Hkv, HD);
        float dot = 0.f;
        for (int i = 0; i < HD; i++) dot = fmaf(sq[i], kp[i], dot);
        s = dot * scale;
      } else {
        s = 0.f;  // unmapped key: zero vector
      }
    }
    const float mx = wave_max(s);
    const float mnew = fmaxf(m, mx);
    const float corr = expf(m - mnew);
    const float p = (j <= g) ? expf(s - mnew) : 0.f;
    l = l * corr + wave_sum(p);
#pragma unroll
    for (int dd = 0; dd < DPL; dd++) acc[dd] *= corr;
    const int nk = min(64, g - j0 + 1);
    for (int kk = 0; kk < nk; kk++) {
      const float pk = __shfl(p, kk, 64);
      const int sk = __shfl(slot, kk, 64);
      if (sk >= 0 && sk < n_slots) {
        const float* vp = v_pool + kv_off(sk, h, Hkv, HD);
#pragma unroll
        for (int dd = 0; dd < DPL; dd++) acc[dd] = fmaf(pk, vp[lane + 64 * dd], acc[dd]);
      }
    }
    m = mnew;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int dd = 0; dd < DPL; dd++) o[((size_t)r * Hq + hq) * HD + lane + 64 * dd] = acc[dd] * inv;
}

// Split count of a bf16 launch: enough (query block, head, split) items to
// fill the chip about twice, at most 16.
int attn_splits(const kvb_model_desc* d, int T_max, int n_cu) {
  const int G = d->n_q_heads / d->n_kv_heads;
  const long items = (long)cdiv(T_max, AQ / G) * d->n_kv_heads;
  const long s = (2L * n_cu + items - 1) / items;
  return (int)(s < 1 ? 1 : (s > 16 ? 16 : s));
}

size_t ws_attn_bytes(const kvb_model_desc* d, int32_t max_rows, int n_cu) {
  if (d->dtype != KVB_BF16) return 0;
  // largest n_split * T over T <= max_rows (n_split shrinks as T grows)
  size_t best = 0;
  const int G = d->n_q_heads / d->n_kv_heads, TB = AQ / G;
  for (int qb = 1; qb <= cdiv(max_rows, TB); qb++) {
    const int T = qb * TB < max_rows ? qb * TB : max_rows;
    const int s = attn_splits(d, T, n_cu);
    if (s == 1) break;
    best = std::max(best, (size_t)s * T);
  }
  if (best == 0) return 0;
  return align_up(best * d->n_q_heads * d->head_dim * 4, 256) + align_up(best * d->n_q_heads * 2 * 4, 256);
}

}  // namespace kvb

using namespace kvb;

extern "C" kvb_status kvb_sparse_query_attn(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                                            const int32_t* n_rows, const int32_t* row_tok, const int32_t* tok_lo,
                                            const void* q, const void* k_pool, const void* v_pool, int32_t n_pages,
                                            const int32_t* slot_map, float scale, void* o, void* ws,
                                            size_t ws_bytes) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0 || n_pages < 0) return fail(KVB_ERR_INVALID_ARG, "T_max or n_pages < 0");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(tok_lo, "tok_lo");
  KVB_CHECK_PTR(q, "q");
  KVB_CHECK_PTR(k_pool, "k_pool");
  KVB_CHECK_PTR(v_pool, "v_pool");
  KVB_CHECK_PTR(slot_map, "slot_map");
  KVB_CHECK_PTR(o, "o");
  if ((long)n_pages * 16 > 0x7fffffffL) return fail(KVB_ERR_INVALID_ARG, "too many pages for int32 slots");
  CtxScope scope(ctx);
  const Ctx* c = current_ctx();
  const int Hq = desc->n_q_heads, Hkv = desc->n_kv_heads, hd = desc->head_dim;
  const int G = Hq / Hkv;
  hipStream_t st = (hipStream_t)stream;
  const int ns = n_pages * 16;
  if (desc->dtype == KVB_BF16) {
    if (G > AQ || AQ % G) return fail(KVB_ERR_UNSUPPORTED, "GQA group size must divide 256");
    const int TB = AQ / G;
    AttnArgs a{};
    a.T_max = T_max;
    a.n_rows = n_rows;
    a.row_tok = row_tok;
    a.tok_lo = tok_lo;
    a.q = (const bf16_t*)q;
    a.k_pool = (const bf16_t*)k_pool;
    a.v_pool = (const bf16_t*)v_pool;
    a.n_slots = ns;
    a.slot_map = slot_map;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.o = (bf16_t*)o;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.n_qblocks = cdiv(T_max, TB);
    // split-KV only when the caller's workspace holds the partials
    int n_split = attn_splits(desc, T_max, c->n_cu);
    const size_t part = align_up((size_t)n_split * T_max * Hq * hd * 4, 256);
    const size_t need = part + align_up((size_t)n_split * T_max * Hq * 2 * 4, 256);
    if (n_split > 1 && (!ws || ws_bytes < need)) n_split = 1;
    a.n_split = n_split;
    if (n_split > 1) {
      a.part_o = (float*)ws;
      a.part_ml = (float*)((char*)ws + part);
    }
    dim3 grid(a.n_qblocks, Hkv, n_split);
    {
      LaunchTimer lt(st, "attention");
      if (hd == 128) attn_bf16_kernel<128><<<grid, ATHREADS, 0, st>>>(a);
      else attn_bf16_kernel<64><<<grid, ATHREADS, 0, st>>>(a);
    }
    KVB_TRY(check_launch("attn_bf16_kernel"));
    if (n_split > 1) {
      LaunchTimer lt(st, "attention_merge");
      const int waves = T_max * Hq;
      if (hd == 128)
        attn_merge_kernel<128><<<cdiv(waves, 4), 256, 0, st>>>(T_max, n_rows, Hq, n_split, a.part_o, a.part_ml,
                                                                (bf16_t*)o);
      else
        attn_merge_kernel<64><<<cdiv(waves, 4), 256, 0, st>>>(T_max, n_rows, Hq, n_split, a.part_o, a.part_ml,
                                                               (bf16_t*)o);
      KVB_TRY(check_launch("attn_merge_kernel"));
    }
    return KVB_OK;
  }
  LaunchTimer lt(st, "attention");
  dim3 grid(T_max, Hq);
  if (hd == 128)
    attn_f32_kernel<128><<<grid, 64, 0, st>>>(T_max, n_rows, row_tok, tok_lo, (const float*)q, (const float*)k_pool,
                                              (const float*)v_pool, ns, slot_map, scale, (float*)o, Hq, Hkv);
  else
    attn_f32_kernel<64><<<grid, 64, 0, st>>>(T_max, n_rows, row_tok, tok_lo, (const float*)q, (const float*)k_pool,
                                             (const float*)v_pool, ns, slot_map, scale, (float*)o, Hq, Hkv);
  return check_launch("attn_f32_kernel");
}
