// Sparse-query causal attention over the paged, spliced KV of one layer
// (EPIC page, section 4, LegoLink steps 3-5: Q of the k' recomputed rows
// against K_exp / V_exp of all N tokens, causal mask, softmax, times V).
//
// bf16 path (gfx950 MFMA, flash-style online softmax):
//   * one block = one KV head x 128 query rows, where a query row is a
//     (token, query head of the GQA group) pair, so the group shares every K/V
//     tile it loads; 4 waves, 32 query rows each;
//   * key tiles of 64 tokens are gathered row by row through the per-token
//     slot map into LDS (register prefetch of the next tile);
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: each lane ends up with 4
//     scores of one query, which is already the operand layout that
//     O^T = V^T P^T needs for P, so probabilities never leave registers;
//   * V tiles are written to LDS transposed (dims x keys), so that V^T
//     operands are plain 8-byte LDS reads;
//   * online softmax statistics live with the lane that owns the query;
//     the mask is lo(row) <= key <= row by global token index;
//   * blocks run longest-first (highest positions first).
// fp32 path: one wave per (row, query head), plain online softmax.
#include "common.h"

namespace kvb {



__device__ __forceinline__ size_t kv_off(int slot, int h, int Hkv, int hd) {
  return (((size_t)(slot >> 4) * Hkv + h) * 16 + (slot & 15)) * hd;
}

constexpr int AQ = 128;        // query rows per block
constexpr int AKT = 64;        // keys per tile
constexpr int ATHREADS = 256;

template <int HD>
__global__ void __launch_bounds__(ATHREADS) attn_bf16_kernel(int T_max, const int32_t* __restrict__ n_rows,
                                                             const int32_t* __restrict__ row_tok,
                                                             const int32_t* __restrict__ tok_lo,
                                                             const bf16_t* __restrict__ q,
                                                             const bf16_t* __restrict__ k_pool,
                                                             const bf16_t* __restrict__ v_pool, int n_slots,
                                                             const int32_t* __restrict__ slot_map, float scale_log2,
                                                             bf16_t* __restrict__ o, int Hq, int Hkv, int n_qblocks) {
  constexpr int LDH = HD + 8;          // LDS row stride (bf16)
  constexpr int KS = HD / 32;          // k slices of the QK^T product
  constexpr int DT = HD / 16;          // 16-wide dim tiles of the PV product
  constexpr int CPR = HD / 8;          // 16-byte chunks per K/V row
  constexpr int LOADS = AKT * CPR / ATHREADS;
  __shared__ __align__(16) bf16_t sK[AKT * LDH];
  constexpr int LDV = AKT + 8;         // keys per row of the transposed V tile
  __shared__ __align__(16) bf16_t sVt[HD * LDV];
  __shared__ int s_kmin, s_kmax;

  const int G = Hq / Hkv;
  const int TB = AQ / G;               // tokens per block
  const int M = row_count(n_rows, T_max);
  const int qb = n_qblocks - 1 - (int)blockIdx.x;  // longest first
  const int h = blockIdx.y;
  const int r0 = qb * TB;
  if (r0 >= M) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  // key range of the block
  if (t == 0) {
    s_kmin = 0x7fffffff;
    s_kmax = -1;
  }
  __syncthreads();
  if (t < TB && r0 + t < M) {
    const int g = row_tok ? row_tok[r0 + t] : r0 + t;
    atomicMin(&s_kmin, tok_lo[g]);
    atomicMax(&s_kmax, g);
  }
  __syncthreads();
  const int kmin = s_kmin, kmax = s_kmax;

  // this lane's two queries (one per 16-wide query tile)
  int qpos[2], qlo[2];
  bool qvalid[2];
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    const int m = wave * 32 + qt * 16 + l16;
    const int r = r0 + m / G, hq = h * G + m % G;
    qvalid[qt] = (m / G) < TB && r < M;
    if (qvalid[qt]) {
      const int g = row_tok ? row_tok[r] : r;
      qpos[qt] = g;
      qlo[qt] = tok_lo[g];
      const bf16_t* qp = q + ((size_t)r * Hq + hq) * HD + g4 * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) qf[qt][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + ks * 32));
    } else {
      qpos[qt] = -1;
      qlo[qt] = 0x7fffffff;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) qf[qt][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
    }
  }

  f32x4_t oacc[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) oacc[dt][0] = oacc[dt][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};

  // K/V tile loaders: chunk c = t + 256 i -> key c / CPR, part c % CPR
  uint4 rk[LOADS], rv[LOADS];
  auto gload = [&](int j0) {
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = t + ATHREADS * i;
      const int key = j0 + c / CPR, part = c % CPR;
      int slot = -1;
      if (key <= kmax) slot = slot_map[key];
      if (slot >= 0 && slot < n_slots) {
        const size_t off = kv_off(slot, h, Hkv, HD) + part * 8;
        rk[i] = *reinterpret_cast<const uint4*>(k_pool + off);
        rv[i] = *reinterpret_cast<const uint4*>(v_pool + off);
      } else {
        rk[i] = rv[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = t + ATHREADS * i;
      const int key = c / CPR, part = c % CPR;
      *reinterpret_cast<uint4*>(sK + key * LDH + part * 8) = rk[i];
      // key k = 32c + 16h + 4g + r sits at column 32c + 8g + 4h + r, so that the 8 keys
      // one lane feeds to the PV product are contiguous
      const int col = (key & 32) | ((key & 12) << 1) | ((key & 16) >> 2) | (key & 3);
      const uint32_t w[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        sVt[(part * 8 + 2 * e) * LDV + col] = (bf16_t)(w[e] & 0xffffu);
        sVt[(part * 8 + 2 * e + 1) * LDV + col] = (bf16_t)(w[e] >> 16);
      }
    }
  };

  const int jstart = kmin;
  if (kmax >= kmin) gload(jstart);
  for (int j0 = jstart; j0 <= kmax; j0 += AKT) {
    __syncthreads();  // previous tile fully consumed
    sstore();
    __syncthreads();
    if (j0 + AKT <= kmax) gload(j0 + AKT);

    // S^T tiles: st[kt][qt] holds keys j0 + 16 kt + 4 g4 + r for query l16 of tile qt
    f32x4_t st[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
      st[kt][0] = st[kt][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(sK + (kt * 16 + l16) * LDH + ks * 32 + g4 * 8));
        st[kt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], st[kt][0], 0, 0, 0);
        st[kt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], st[kt][1], 0, 0, 0);
      }
    }
    // mask, online softmax (statistics per query; each query is spread over 4 lanes: xor 16, 32).
    // Scores are copied out of the MFMA result vectors into plain floats first.
    bf16x8_t pf[2][2];  // [qt][key half]: B operand of the PV product
#pragma unroll
    for (int qt = 0; qt < 2; qt++) {
      float sv[16];
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
        const f32x4_t a = st[kt][qt];
        sv[kt * 4 + 0] = a[0];
        sv[kt * 4 + 1] = a[1];
        sv[kt * 4 + 2] = a[2];
        sv[kt * 4 + 3] = a[3];
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int key = j0 + (i >> 2) * 16 + g4 * 4 + (i & 3);
        const bool ok = key <= qpos[qt] && key >= qlo[qt];
        sv[i] = ok ? sv[i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qt], mx);
      const bool dead = mnew == -INFINITY;
      const float corr = dead ? 1.f : exp2f(mrow[qt] - mnew);
      mrow[qt] = mnew;
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        sv[i] = dead ? 0.f : exp2f(sv[i] - mnew);
        ls += sv[i];
      }
      lrow[qt] = lrow[qt] * corr + ls;
      {
        // (a splat-vector product: the scalar form trips a backend crash in this toolchain)
        const f32x4_t cv = {corr, corr, corr, corr};
#pragma unroll
        for (int dt = 0; dt < DT; dt++) oacc[dt][qt] = oacc[dt][qt] * cv;
      }
#pragma unroll
      for (int c = 0; c < 2; c++) {
        uint4 w;
        w.x = (uint32_t)f2bf(sv[8 * c + 0]) | ((uint32_t)f2bf(sv[8 * c + 1]) << 16);
        w.y = (uint32_t)f2bf(sv[8 * c + 2]) | ((uint32_t)f2bf(sv[8 * c + 3]) << 16);
        w.z = (uint32_t)f2bf(sv[8 * c + 4]) | ((uint32_t)f2bf(sv[8 * c + 5]) << 16);
        w.w = (uint32_t)f2bf(sv[8 * c + 6]) | ((uint32_t)f2bf(sv[8 * c + 7]) << 16);
        pf[qt][c] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    // O^T += V^T P^T: A operand of lane l = V[the keys of its k slots][dim dt*16 + l16],
    // one 16-byte read from the transposed, key-permuted V tile
#pragma unroll
    for (int c = 0; c < 2; c++) {
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(sVt + (dt * 16 + l16) * LDV + 32 * c + 8 * g4));
        oacc[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[0][c], oacc[dt][0], 0, 0, 0);
        oacc[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[1][c], oacc[dt][1], 0, 0, 0);
      }
    }
  }

  // normalise and store: oacc[dt][qt][r] = O[query l16 of tile qt][dim dt*16 + 4 g4 + r]
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    float l = lrow[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!qvalid[qt]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int m = wave * 32 + qt * 16 + l16;
    const int r = r0 + m / G, hq = h * G + m % G;
    bf16_t* op = o + ((size_t)r * Hq + hq) * HD;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      uint2 w;
      w.x = (uint32_t)f2bf(oacc[dt][qt][0] * inv) | ((uint32_t)f2bf(oacc[dt][qt][1] * inv) << 16);
      w.y = (uint32_t)f2bf(oacc[dt][qt][2] * inv) | ((uint32_t)f2bf(oacc[dt][qt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + dt * 16 + 4 * g4) = w;
    }
  }
}

// ------------------------------------------------------------------ fp32 reference-style kernel
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

}  // namespace kvb

using namespace kvb;

extern "C" kvb_status kvb_sparse_query_attn(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                                            const int32_t* n_rows, const int32_t* row_tok, const int32_t* tok_lo,
                                            const void* q, const void* k_pool, const void* v_pool, int32_t n_pages,
                                            const int32_t* slot_map, float scale, void* o, void* ws,
                                            size_t ws_bytes) {
  (void)ws;
  (void)ws_bytes;
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
  const int Hq = desc->n_q_heads, Hkv = desc->n_kv_heads, hd = desc->head_dim;
  const int G = Hq / Hkv;
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  const int ns = n_pages * 16;
  LaunchTimer lt(st, "attention");
  if (desc->dtype == KVB_BF16) {
    if (G > AQ || AQ % G) return fail(KVB_ERR_UNSUPPORTED, "GQA group size must divide 128");
    const int TB = AQ / G;
    const int nqb = cdiv(T_max, TB);
    dim3 grid(nqb, Hkv);
    const float sl2 = scale * 1.4426950408889634f;
    if (hd == 128)
      attn_bf16_kernel<128><<<grid, ATHREADS, 0, st>>>(T_max, n_rows, row_tok, tok_lo, (const bf16_t*)q,
                                                       (const bf16_t*)k_pool, (const bf16_t*)v_pool, ns, slot_map,
                                                       sl2, (bf16_t*)o, Hq, Hkv, nqb);
    else
      attn_bf16_kernel<64><<<grid, ATHREADS, 0, st>>>(T_max, n_rows, row_tok, tok_lo, (const bf16_t*)q,
                                                      (const bf16_t*)k_pool, (const bf16_t*)v_pool, ns, slot_map, sl2,
                                                      (bf16_t*)o, Hq, Hkv, nqb);
    return check_launch("attn_bf16_kernel");
  }
  dim3 grid(T_max, Hq);
  if (hd == 128)
    attn_f32_kernel<128><<<grid, 64, 0, st>>>(T_max, n_rows, row_tok, tok_lo, (const float*)q, (const float*)k_pool,
                                              (const float*)v_pool, ns, slot_map, scale, (float*)o, Hq, Hkv);
  else
    attn_f32_kernel<64><<<grid, 64, 0, st>>>(T_max, n_rows, row_tok, tok_lo, (const float*)q, (const float*)k_pool,
                                             (const float*)v_pool, ns, slot_map, scale, (float*)o, Hq, Hkv);
  return check_launch("attn_f32_kernel");
}
