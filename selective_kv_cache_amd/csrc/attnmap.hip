// Attention-map deviation of the CacheBlend-style selection (EPIC page,
// section 3.2, the CacheBlend baseline: once layer 1 is recomputed for every
// token, each token's attention map under the cached keys is compared with its
// map under the recomputed keys, and the tokens that differ most are the ones
// recomputed in the later layers).
//
//   dev[g] = (1 / Hq) sum_h sum_{j = lo[g] .. g} | Pn[h, g, j] - Po[h, g, j] |
//   Pn[h, g, :] = softmax_j(q[g, h] . k_rec[j, h / G] * scale)
//   Po[h, g, :] = softmax_j(q[g, h] . k_pool[reuse_slot[j], h / G] * scale)
//
// bf16 path (gfx950 MFMA):
//   * one block = one KV head x 256 query rows, a query row being a (token,
//     query head of the GQA group) pair, so the group shares every key tile;
//     8 waves x 32 query rows;
//   * two passes over the block's key range: the first keeps the running
//     maximum and sum of both rows (online softmax), the second adds the
//     distance of the normalised rows; both passes compute the scores with the
//     same instructions, so the statistics match the probabilities exactly;
//   * key tiles of 64 tokens, the recomputed keys read by token and the cached
//     keys gathered through the reuse slots, land in LDS by direct-to-LDS
//     loads one tile ahead; the slot indices arrive the same way one tile
//     before the keys;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16, once per map: a lane ends with
//     16 scores of one query, so the row statistics need one xor-32 exchange;
//   * the group's heads of a token sit in adjacent lanes and are summed there;
//     per KV head the block writes one partial per token, which a second
//     kernel adds in a fixed order (bitwise deterministic).
// A key whose reuse slot is outside the pool is left out of both maps.
// fp32 path: one block per token, one wave per query head at a time, plain
// two-pass softmax.
#include "common.h"

// No implicit multiply-add contraction in this file: every fused operation is
// written out and applied to both maps alike, so equal scores give exactly 0.
#pragma clang fp contract(off)

namespace kvb {

constexpr int MQ = 256;        // query rows per block
constexpr int MKT = 64;        // keys per tile
constexpr int MWAVES = 8;      // 32 query rows each
constexpr int MTHREADS = 64 * MWAVES;

struct MapArgs {
  int n_tok;
  const int32_t* tok_lo;
  const bf16_t* q;       // [n_tok, Hq, HD]
  const bf16_t* k_rec;   // [n_tok, Hkv, HD]
  const bf16_t* k_pool;  // [pages, Hkv, 16, HD]
  int n_slots;
  const int32_t* reuse_slot;
  float scale_log2;
  float* partial;        // [Hkv, n_tok]
  int Hq, Hkv, n_qblocks;
};

// key tile geometry in LDS: 64 rows of HD bf16, row-major, 16-byte chunk c of
// row r stored at chunk position c ^ swz(r); one direct-to-LDS instruction
// fills 1 KiB = RPI rows, wave w fills rows 8 w .. 8 w + 7
template <int HD>
struct MapGeom {
  static constexpr int ROWB = HD * 2;
  static constexpr int CPR = HD / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int TILE = MKT * ROWB;
  static constexpr int IPW = TILE / 1024 / MWAVES;
  static constexpr int STAGE = 2 * TILE;  // recomputed tile, then cached tile
  // the fragment read of 16 consecutive rows at one chunk hits 16 distinct bank groups
  __device__ __forceinline__ static int swz(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
};

template <int HD>
__global__ void __launch_bounds__(MTHREADS) __attribute__((amdgpu_waves_per_eu(4, 4))) attnmap_bf16_kernel(MapArgs a) {
  using Gm = MapGeom<HD>;
  constexpr int KS = HD / 16;
  constexpr int ROWB = Gm::ROWB, CPR = Gm::CPR, RPI = Gm::RPI, IPW = Gm::IPW, TILE = Gm::TILE;
  static_assert(IPW * RPI == 8, "a wave loads 8 key rows");
  __shared__ __align__(16) uint8_t s_kv[2 * Gm::STAGE];
  __shared__ __align__(16) int32_t s_slot[2][MWAVES][64];  // per stage, wave: keys 8 w + (lane % 8)
  __shared__ __align__(8) uint8_t s_inval[2][MWAVES];      // invalid-slot bits of each wave's 8 keys
  __shared__ int s_kmin, s_kmax, s_pmin, s_lomax;

  const int G = a.Hq / a.Hkv;
  const int TB = MQ / G;  // tokens per block
  const int qb = a.n_qblocks - 1 - (int)blockIdx.x;  // longest first
  const int h = blockIdx.y;
  const int r0 = qb * TB;
  if (r0 >= a.n_tok) return;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;

  if (t == 0) {
    s_kmin = 0x7fffffff;
    s_kmax = -1;
    s_pmin = 0x7fffffff;
    s_lomax = -1;
  }
  __syncthreads();
  if (t < TB && r0 + t < a.n_tok) {
    const int g = r0 + t;
    const int lo = a.tok_lo[g];
    atomicMin(&s_kmin, lo);
    atomicMax(&s_kmax, g);
    atomicMin(&s_pmin, g);
    atomicMax(&s_lomax, lo);
  }
  __syncthreads();
  const int kmin = s_kmin, kmax = s_kmax, pmin = s_pmin, lomax = s_lomax;
  const int nt = (kmax - kmin) / MKT + 1;

  // this lane's query: column l32 of the wave's 32 query rows
  const int m = wave * 32 + l32;
  const int r = r0 + m / G, hq = h * G + m % G;
  const bool qvalid = r < a.n_tok;
  int qpos = -1, qlo = 0x7fffffff;
  bf16x8_t qf[KS];
  if (qvalid) {
    qpos = r;
    qlo = a.tok_lo[r];
    const bf16_t* qp = a.q + ((size_t)r * a.Hq + hq) * HD + g2 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + ks * 16));
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ks++) qf[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
  }
  // K fragment of (half kt, step ks): row 32 kt + l32, chunk 2 ks + g2
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) koff[ks] = l32 * ROWB + (((2 * ks + g2) ^ Gm::swz(l32)) * 16);
  // the query loads complete here: no load the compiler tracks is left for the loops
  wait_vmcnt<0>();

  // slot indices of tile X's 8 keys of this wave -> s_slot[X % 2][wave]
  auto issue_slots = [&](int X) {
    int key = kmin + X * MKT + wave * 8 + (lane & 7);
    key = key < kmax ? key : kmax;  // keys past the block's last query are masked anyway
    dma4(a.reuse_slot + key, __builtin_amdgcn_readfirstlane(lds_addr(&s_slot[X & 1][wave][0])));
  };
  // recomputed and cached rows of tile X's 8 keys of this wave; needs s_slot[X % 2][wave]
  auto issue_kv = [&](int X) {
    const int st = X & 1;
    uint8_t* nb = s_kv + st * Gm::STAGE;
    uint8_t* ob = nb + TILE;
    uint32_t bad = 0;
#pragma unroll
    for (int i = 0; i < IPW; i++) {
      const int rl = i * RPI + lane / CPR;
      const int row = wave * 8 + rl;
      int key = kmin + X * MKT + row;
      key = key < kmax ? key : kmax;
      int slot = s_slot[st][wave][rl];
      const bool ok = (unsigned)slot < (unsigned)a.n_slots;
      const uint64_t bb = __ballot(!ok);
      if (bb) {
#pragma unroll
        for (int u = 0; u < RPI; u++) bad |= (uint32_t)((bb >> (u * CPR)) & 1u) << (i * RPI + u);
      }
      slot = ok ? slot : 0;
      const uint32_t prow = (uint32_t)(slot >> 4) * (uint32_t)(a.Hkv * 16) + (uint32_t)(h * 16 + (slot & 15));
      const int chunk = (lane % CPR) ^ Gm::swz(row);
      const uint32_t dst = (uint32_t)(wave * IPW + i) * 1024u;
      dma16(a.k_rec + ((size_t)key * a.Hkv + h) * HD + chunk * 8, __builtin_amdgcn_readfirstlane(lds_addr(nb + dst)));
      dma16(a.k_pool + (size_t)prow * HD + chunk * 8, __builtin_amdgcn_readfirstlane(lds_addr(ob + dst)));
    }
    if (lane == 0) s_inval[st][wave] = (uint8_t)bad;
  };

  // running statistics of the query's two rows (base-2 units); in pass 2 the
  // final offsets and reciprocal sums
  float mn = -INFINITY, ln = 0.f, mo = -INFINITY, lo_ = 0.f;
  float inv_n = 0.f, ratio = 0.f, acc = 0.f;

  for (int pass = 0; pass < 2; pass++) {
    // prologue: slots of tiles 0 and 1, keys of tile 0
    issue_slots(0);
    wait_vmcnt<0>();
    issue_kv(0);
    if (nt > 1) issue_slots(1);
    for (int X = 0; X < nt; X++) {
      // keys of tile X complete; slots of tile X + 1 may still be in flight
      if (X + 1 < nt) wait_vmcnt<1>();
      else wait_vmcnt<0>();
      lds_barrier();  // tile X published; every wave is done with tile X - 1
      if (X + 1 < nt) {
        wait_vmcnt<0>();
        issue_kv(X + 1);
        if (X + 2 < nt) issue_slots(X + 2);
      }
      const int st = X & 1;
      const uint8_t* nbs = s_kv + st * Gm::STAGE;
      const uint8_t* obs = nbs + TILE;
      const int j0 = kmin + X * MKT;
      const uint64_t inval = *reinterpret_cast<const uint64_t*>(&s_inval[st][0]);
      const bool need_mask = (j0 + MKT - 1 > pmin) || (j0 < lomax) || inval != 0;
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        f32x16_t sn = (f32x16_t){}, so = (f32x16_t){};
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          const bf16x8_t kn = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(nbs + kt * 32 * ROWB + koff[ks]));
          const bf16x8_t ko = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(obs + kt * 32 * ROWB + koff[ks]));
          sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kn, qf[ks], sn, 0, 0, 0);
          so = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ko, qf[ks], so, 0, 0, 0);
        }
        // raw scores of keys j0 + 32 kt + 8 (r / 4) + 4 g2 + r % 4; a probability is
        // exp2(fma(score, scale_log2, -offset)) with the row's base-2 offset
        float tn[16], to[16];
#pragma unroll
        for (int e = 0; e < 16; e++) {
          tn[e] = sn[e];
          to[e] = so[e];
        }
        if (need_mask) {
          const uint32_t iv = (uint32_t)(inval >> (kt * 32 + 4 * g2));
#pragma unroll
          for (int e = 0; e < 16; e++) {
            const int key = j0 + kt * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
            if (key > qpos || key < qlo || ((iv >> (8 * (e >> 2) + (e & 3))) & 1u)) {
              tn[e] = -INFINITY;
              to[e] = -INFINITY;
            }
          }
        }
        const float c = a.scale_log2;
        if (pass == 0) {
          float xn = tn[0], xo = to[0];
#pragma unroll
          for (int e = 1; e < 16; e++) {
            xn = fmaxf(xn, tn[e]);
            xo = fmaxf(xo, to[e]);
          }
          xn = fmaxf(xn, __shfl_xor(xn, 32, 64)) * c;
          xo = fmaxf(xo, __shfl_xor(xo, 32, 64)) * c;
          if (xn > mn) {
            ln *= __builtin_amdgcn_exp2f(mn - xn);
            mn = xn;
          }
          if (xo > mo) {
            lo_ *= __builtin_amdgcn_exp2f(mo - xo);
            mo = xo;
          }
          if (mn != -INFINITY) {
#pragma unroll
            for (int e = 0; e < 16; e++) ln += __builtin_amdgcn_exp2f(fmaf(tn[e], c, -mn));
          }
          if (mo != -INFINITY) {
#pragma unroll
            for (int e = 0; e < 16; e++) lo_ += __builtin_amdgcn_exp2f(fmaf(to[e], c, -mo));
          }
        } else {
          // |pn - po| = inv_n |en - ratio eo|, ratio = ln / lo (exactly 1 for equal rows)
#pragma unroll
          for (int e = 0; e < 16; e++) {
            const float en = __builtin_amdgcn_exp2f(fmaf(tn[e], c, -mn));
            const float eo = __builtin_amdgcn_exp2f(fmaf(to[e], c, -mo));
            acc += fabsf(fmaf(-eo, ratio, en));
          }
        }
      }
    }
    if (pass == 0) {
      // both lanes of a query hold the same offsets; the sums add across them
      ln += __shfl_xor(ln, 32, 64);
      lo_ += __shfl_xor(lo_, 32, 64);
      inv_n = ln > 0.f ? 1.f / ln : 0.f;
      ratio = lo_ > 0.f ? ln / lo_ : 0.f;
      if (mn == -INFINITY) mn = 0.f;  // no visible key: every probability is 0
      if (mo == -INFINITY) mo = 0.f;
      lds_barrier();  // every wave is done with the last tile before pass 2 refills stage 0
    }
  }
  acc *= inv_n;
  // the query's two halves, then the group's heads (adjacent lanes)
  acc += __shfl_xor(acc, 32, 64);
  for (int o = 1; o < G; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (qvalid && g2 == 0 && (l32 % G) == 0) a.partial[(size_t)h * a.n_tok + r] = acc;
}

// dev[g] = (sum over KV heads of partial[h][g]) / Hq, heads in order
__global__ void attnmap_reduce_kernel(int n_tok, int Hkv, int Hq, const float* __restrict__ partial,
                                      float* __restrict__ dev) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_tok) return;
  float s = 0.f;
  for (int h = 0; h < Hkv; h++) s += partial[(size_t)h * n_tok + g];
  dev[g] = s / (float)Hq;
}

// ------------------------------------------------------------------ fp32 kernel
// one block per token; each wave takes query heads wave, wave + 4, ...; one key per lane

constexpr int FWAVES = 4;
constexpr int FMAXH = 256;

__device__ __forceinline__ size_t map_pool_off(int slot, int h, int Hkv, int hd) {
  return (((size_t)(slot >> 4) * Hkv + h) * 16 + (slot & 15)) * hd;
}

template <int HD>
__global__ void __launch_bounds__(64 * FWAVES) attnmap_f32_kernel(int n_tok, const int32_t* __restrict__ tok_lo,
                                                                  const float* __restrict__ q,
                                                                  const float* __restrict__ k_rec,
                                                                  const float* __restrict__ k_pool, int n_slots,
                                                                  const int32_t* __restrict__ reuse_slot, float scale,
                                                                  float* __restrict__ dev, int Hq, int Hkv) {
  __shared__ float sq[FWAVES][HD];
  __shared__ float s_head[FMAXH];
  const int g = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lo = tok_lo[g];
  const int G = Hq / Hkv;
  for (int base = 0; base < Hq; base += FWAVES) {
    const int hq = base + wave;
    const int h = hq / G;
    __syncthreads();  // the previous iteration's reads of sq are done
    if (hq < Hq)
      for (int i = lane; i < HD; i += 64) sq[wave][i] = q[((size_t)g * Hq + hq) * HD + i];
    __syncthreads();
    if (hq >= Hq) continue;
    // scores of key j under both maps (-inf: not visible)
    auto scores = [&](int j, float& s_n, float& s_o) {
      s_n = -INFINITY;
      s_o = -INFINITY;
      if (j > g) return;
      const int slot = reuse_slot[j];
      if (slot < 0 || slot >= n_slots) return;
      const float* kn = k_rec + ((size_t)j * Hkv + h) * HD;
      const float* ko = k_pool + map_pool_off(slot, h, Hkv, HD);
      float dn = 0.f, dn_o = 0.f;
      for (int i = 0; i < HD; i++) {
        dn = fmaf(sq[wave][i], kn[i], dn);
        dn_o = fmaf(sq[wave][i], ko[i], dn_o);
      }
      s_n = dn * scale;
      s_o = dn_o * scale;
    };
    float mn = -INFINITY, mo = -INFINITY;
    for (int j0 = lo; j0 <= g; j0 += 64) {
      float a, b;
      scores(j0 + lane, a, b);
      mn = fmaxf(mn, a);
      mo = fmaxf(mo, b);
    }
    mn = wave_max(mn);
    mo = wave_max(mo);
    if (mn == -INFINITY) mn = 0.f;  // no visible key: every probability is 0
    if (mo == -INFINITY) mo = 0.f;
    float ln = 0.f, lo_ = 0.f;
    for (int j0 = lo; j0 <= g; j0 += 64) {
      float a, b;
      scores(j0 + lane, a, b);
      ln += expf(a - mn);
      lo_ += expf(b - mo);
    }
    ln = wave_sum(ln);
    lo_ = wave_sum(lo_);
    const float inv_n = ln > 0.f ? 1.f / ln : 0.f, inv_o = lo_ > 0.f ? 1.f / lo_ : 0.f;
    float acc = 0.f;
    for (int j0 = lo; j0 <= g; j0 += 64) {
      float a, b;
      scores(j0 + lane, a, b);
      acc += fabsf(expf(a - mn) * inv_n - expf(b - mo) * inv_o);
    }
    acc = wave_sum(acc);
    if (lane == 0) s_head[hq] = acc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int hq = 0; hq < Hq; hq++) s += s_head[hq];
    dev[g] = s / (float)Hq;
  }
}

size_t ws_attnmap_bytes(const kvb_model_desc* d, int32_t max_tokens) {
  if (d->dtype != KVB_BF16) return 0;
  return align_up((size_t)d->n_kv_heads * (size_t)max_tokens * 4, 256);
}

}  // namespace kvb

using namespace kvb;

extern "C" kvb_status kvb_attnmap_deviation(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t n_tok,
                                            const int32_t* tok_lo, const void* q, const void* k_rec,
                                            const void* k_pool, int32_t n_pages, const int32_t* reuse_slot,
                                            float scale, float* dev, void* ws, size_t ws_bytes) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (n_tok < 0 || n_pages < 0) return fail(KVB_ERR_INVALID_ARG, "negative size");
  if (n_tok == 0) return KVB_OK;
  KVB_CHECK_PTR(tok_lo, "tok_lo");
  KVB_CHECK_PTR(q, "q");
  KVB_CHECK_PTR(k_rec, "k_rec");
  KVB_CHECK_PTR(k_pool, "k_pool");
  KVB_CHECK_PTR(reuse_slot, "reuse_slot");
  KVB_CHECK_PTR(dev, "dev");
  const int Hq = desc->n_q_heads, Hkv = desc->n_kv_heads, hd = desc->head_dim;
  const int G = Hq / Hkv;
  if (hd != 64 && hd != 128) return fail(KVB_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if ((long)n_pages * 16 > 0x7fffffffL) return fail(KVB_ERR_INVALID_ARG, "pool too large for int32 slots");
  if (desc->dtype == KVB_BF16) {
    if (G > 32 || (G & (G - 1)) != 0)
      return fail(KVB_ERR_UNSUPPORTED, "n_q_heads / n_kv_heads must be a power of two up to 32");
    if (!ws || ws_bytes < ws_attnmap_bytes(desc, n_tok))
      return fail(KVB_ERR_WORKSPACE, "kvb_attnmap_deviation workspace too small");
  } else if (Hq > FMAXH) {
    return fail(KVB_ERR_UNSUPPORTED, "n_q_heads > 256 on the float32 path");
  }
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  if (desc->dtype == KVB_BF16) {
    MapArgs a;
    a.n_tok = n_tok;
    a.tok_lo = tok_lo;
    a.q = (const bf16_t*)q;
    a.k_rec = (const bf16_t*)k_rec;
    a.k_pool = (const bf16_t*)k_pool;
    a.n_slots = n_pages * 16;
    a.reuse_slot = reuse_slot;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.partial = (float*)ws;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.n_qblocks = cdiv(n_tok, MQ / G);
    dim3 grid(a.n_qblocks, Hkv);
    {
      LaunchTimer lt(st, "attnmap");
      if (hd == 128) attnmap_bf16_kernel<128><<<grid, MTHREADS, 0, st>>>(a);
      else attnmap_bf16_kernel<64><<<grid, MTHREADS, 0, st>>>(a);
    }
    KVB_TRY(check_launch("attnmap_bf16_kernel"));
    {
      LaunchTimer lt(st, "attnmap_reduce");
      attnmap_reduce_kernel<<<cdiv(n_tok, 256), 256, 0, st>>>(n_tok, Hkv, Hq, a.partial, dev);
    }
    return check_launch("attnmap_reduce_kernel");
  }
  {
    LaunchTimer lt(st, "attnmap");
    if (hd == 128)
      attnmap_f32_kernel<128><<<n_tok, 64 * FWAVES, 0, st>>>(n_tok, tok_lo, (const float*)q, (const float*)k_rec,
                                                               (const float*)k_pool, n_pages * 16, reuse_slot, scale,
                                                               dev, Hq, Hkv);
    else
      attnmap_f32_kernel<64><<<n_tok, 64 * FWAVES, 0, st>>>(n_tok, tok_lo, (const float*)q, (const float*)k_rec,
                                                              (const float*)k_pool, n_pages * 16, reuse_slot, scale,
                                                              dev, Hq, Hkv);
  }
  return check_launch("attnmap_f32_kernel");
}
