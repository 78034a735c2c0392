// Sparse-query causal attention over the paged, spliced KV of one layer
// (EPIC page, section 4, LegoLink steps 3-5: Q of the k' recomputed rows
// against K_exp / V_exp of all N tokens, causal mask, softmax, times V).
//
// bf16 path (gfx950 MFMA, flash-style online softmax):
//   * one block = one KV head x 256 query rows, a query row being a (token,
//     query head of the GQA group) pair, so the whole group shares every K/V
//     tile; 8 waves x 32 query rows, two waves per SIMD;
//   * key tiles of 64 tokens are gathered through the per-token slot map by
//     direct-to-LDS loads into a 3-stage ring, two tiles ahead;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane ends with 16 scores of
//     one query, which is already the B-operand layout of O^T = V^T P^T, so
//     probabilities stay in registers; softmax statistics need one xor-32
//     exchange per query (a lane-half swap, not an LDS permute);
//   * V stays row-major in LDS; V^T operands come from the transposing LDS
//     read of gfx950;
//   * only tiles that cross a query's causal edge or its lower bound, or that
//     hold a key without a valid slot, are masked; blocks run longest first,
//     each XCD taking whole KV heads so its L2 holds the K/V its blocks share;
//   * split-KV: with few query blocks the key range of each block is cut into
//     n_split parts whose partial (O, offset, sum) a merge kernel combines.
// fp32 path: one wave per (row, query head), plain online softmax.
#include "common.h"

#include <type_traits>

namespace kvb {

__device__ __forceinline__ size_t kv_off(int slot, int h, int Hkv, int hd) {
  return (((size_t)(slot >> 4) * Hkv + h) * 16 + (slot & 15)) * hd;
}

constexpr int AQ = 256;        // query rows per block
constexpr int AKT = 64;        // keys per tile
constexpr int ANST = 3;        // LDS ring stages (tiles in flight: 2 ahead)
constexpr int AWAVES = 8;      // 32 query rows each
constexpr int ATHREADS = 64 * AWAVES;

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

// K / V tile geometry in LDS: 64 key rows of HD bf16, row-major, the 16-byte
// chunk c of row r stored at chunk position c ^ swizzle(r).  One direct-to-LDS
// instruction fills 1 KiB = RPI rows; wave w fills rows 8 w .. 8 w + 7.
template <int HD>
struct AttnGeom {
  static constexpr int ROWB = HD * 2;                // bytes per key row
  static constexpr int CPR = HD / 8;                 // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;               // rows per 1 KiB instruction
  static constexpr int TILE = AKT * ROWB;            // bytes of one K (or V) tile
  static constexpr int IPW = TILE / 1024 / AWAVES;   // instructions per wave per tile
  static constexpr int STAGE = 2 * TILE;             // one K and one V tile
  // K: the fragment read of 16 consecutive rows at one chunk hits 16 distinct
  // bank groups.  V: the transposing read of 4 consecutive rows x 4 chunks
  // hits 16 distinct bank groups.  Both depend on the low row bits only.
  __device__ __forceinline__ static int swz_k(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ __forceinline__ static int swz_v(int r) { return HD == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// this lane's index, recomputed where it is needed: a kept copy would hold a
// register through the whole loop
__device__ __forceinline__ int lane_id_opaque() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// max of v over lanes l and l ^ 32 without an LDS round trip: the half swap of
// gfx950 leaves one half of v in both halves of one result and the other half
// in both halves of the other
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// gfx950 transposing LDS read: in every 16-lane group, lane i receives element
// i % 4 of the 8 bytes addressed by lanes i / 4 + 4 s of the group, s = 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Block: one KV head x AQ query rows, a query row being a (token, query head of
// the GQA group) pair; 8 waves x 32 rows.  At most 256 registers per wave, so
// two waves share a SIMD and one's MFMAs overlap the other's softmax.
//
// Per 64-key tile (ring stage X % 3), in two 32-key halves:
//   S^T = K Q^T       v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q held
//                     in registers; a lane ends with 16 scores of one query
//                     (keys 8 (r / 4) + 4 (lane / 32) + r % 4 of the half);
//   softmax           base 2, scale folded into one FMA; the running offset
//                     m only moves (and O is rescaled) when a half's maximum
//                     exceeds it by more than 8, so rescales are rare;
//   O^T += V^T P^T    P^T is the lane's own scores (bf16) with the key order
//                     of each 16-key step permuted the same way on both sides;
//                     V^T fragments come from the row-major V tile through the
//                     transposing LDS read.
// Tiles are gathered through the per-token slot map by direct-to-LDS loads two
// tiles ahead; the slot indices of a tile arrive the same way one tile earlier,
// so no load the compiler can see is waited on inside the loop.  A key whose
// slot is outside the pool is excluded from every row's softmax.
template <int HD>
__global__ void __launch_bounds__(ATHREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_kernel(AttnArgs a) {
  using Gm = AttnGeom<HD>;
  constexpr int KS = HD / 16;  // k16 steps of Q K^T
  constexpr int DT = HD / 32;  // 32-wide dim tiles of P V
  constexpr int ROWB = Gm::ROWB, CPR = Gm::CPR, RPI = Gm::RPI, IPW = Gm::IPW, TILE = Gm::TILE;
  static_assert(IPW * RPI == 8, "a wave loads 8 key rows");
  __shared__ __align__(16) uint8_t s_kv[ANST * Gm::STAGE];
  __shared__ __align__(16) int32_t s_slot[ANST][AWAVES][64];  // per stage, wave: keys 8 w + (lane % 8)
  // invalid-slot bits of each wave's 8 keys, one byte per wave: a stage's 64
  // bits read back as one word
  __shared__ __align__(8) uint8_t s_inval[ANST][AWAVES];
  static_assert(AWAVES == 8, "one byte per wave makes the 64-key word");
  __shared__ int s_kmin, s_kmax, s_pmin, s_lomax;

  const int G = a.Hq / a.Hkv;
  const int TB = AQ / G;  // tokens per block
  const int M = row_count(a.n_rows, a.T_max);
  // Workgroups go to the 8 XCDs round-robin by id, each XCD with its own L2
  // (4 MiB, about the K/V of one head over 8K tokens): give every XCD whole KV
  // heads (or every head a fixed set of XCDs), so the K/V rows a block streams
  // are the ones the other blocks on its XCD stream too.
  int h, item;
  {
    const int L = blockIdx.x, xcd = L & 7, i = L >> 3;
    const int per_head = a.n_qblocks * a.n_split;
    if (a.Hkv % 8 == 0) {
      const int hp = a.Hkv / 8;
      h = xcd * hp + i % hp;
      item = i / hp;
    } else if (8 % a.Hkv == 0) {
      const int xp = 8 / a.Hkv;
      h = xcd / xp;
      item = i * xp + xcd % xp;
    } else {
      h = L / per_head;
      item = L % per_head;
    }
    if (h >= a.Hkv || item >= per_head) return;
  }
  const int qb = a.n_qblocks - 1 - item / a.n_split;  // longest first
  const int split = item % a.n_split;
  const int r0 = qb * TB;
  if (r0 >= M) return;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, g2 = lane >> 5, l16 = lane & 15;

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
  const int nt = (int)((long)ntiles * (split + 1) / a.n_split) - t_begin;
  const int kbase = kmin + t_begin * AKT;  // first key of tile 0

  // this lane's query: column l32 of the wave's query tile
  int qpos, qlo;
  bool qvalid;
  bf16x8_t qf[KS];
  {
    const int m = wave * 32 + l32;
    const int r = r0 + m / G, hq = h * G + m % G;
    qvalid = r < M;
    if (qvalid) {
      const int g = a.row_tok ? a.row_tok[r] : r;
      qpos = g;
      qlo = a.tok_lo[g];
      const bf16_t* qp = a.q + ((size_t)r * a.Hq + hq) * HD + g2 * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + ks * 16));
    } else {
      qpos = -1;
      qlo = 0x7fffffff;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) qf[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
    }
  }

  // per-lane LDS byte offsets of the fragment reads inside a stage:
  //   K fragment (half kt, step ks): row 32 kt + l32, chunk 2 ks + g2
  //   V^T fragment (step c, dims 32 dt, part u): source row 16 c + 8 u + 4 g2 + l16 / 4,
  //     dims 32 dt + 16 ((lane / 16) % 2) + 4 (l16 % 4) .. + 3
  // the swizzles depend on the low row bits only, so kt, c and u are immediates.
  int koff[KS], voff[DT];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    koff[ks] = l32 * ROWB + (((2 * ks + g2) ^ Gm::swz_k(l32)) * 16);
    // opaque, so stage + half offsets stay immediates of the reads rather
    // than being merged into the lane offset with a per-read OR
    asm volatile("" : "+v"(koff[ks]));
  }
  {
    const int vr = 4 * g2 + (l16 >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      const int chunk = 4 * dt + 2 * ((lane >> 4) & 1) + ((l16 >> 1) & 1);
      // V tiles start after the ANST K tiles; the base is folded in here and
      // hidden from the compiler so the stage offset stays an immediate
      voff[dt] = ANST * TILE + vr * ROWB + ((chunk ^ Gm::swz_v(vr)) * 16) + 8 * (l16 & 1);
      asm volatile("" : "+v"(voff[dt]));
    }
  }

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) oacc[dt] = (f32x16_t){};
  float moff = -INFINITY, lrow = 0.f;
  // the query loads complete here, so the compiler has no load of its own to
  // wait for inside the loop (such a wait would also drain the K/V ring)
  wait_vmcnt<0>();

  // The per-lane parts of the load addresses are recomputed at every issue from
  // the lane index: hoisted out of the loop they would take registers for the
  // whole loop.
  // slot indices of tile X's 8 keys of this wave -> s_slot[X % 3][wave] (1 load per lane)
  auto issue_slots = [&](int X) {
    const int ln = lane_id_opaque();
    int key = kbase + X * AKT + wave * 8 + (ln & 7);
    key = key < kmax ? key : kmax;  // keys past the block's last query are masked anyway
    dma4(a.slot_map + key, __builtin_amdgcn_readfirstlane(lds_addr(&s_slot[X % ANST][wave][0])));
  };
  // K and V rows of tile X's 8 keys of this wave (2 IPW loads per lane); needs
  // s_slot[X % 3][wave] complete
  auto issue_kv = [&](int X) {
    const int st = X % ANST;
    uint8_t* kb = s_kv + st * TILE;
    uint8_t* vb = s_kv + (ANST + st) * TILE;
    uint32_t bad = 0;
    const int ln = lane_id_opaque();
#pragma unroll
    for (int i = 0; i < IPW; i++) {
      const int rl = i * RPI + ln / CPR;  // row among the wave's 8
      const int row = wave * 8 + rl;
      int slot = s_slot[st][wave][rl];
      const bool ok = (unsigned)slot < (unsigned)a.n_slots;
      const uint64_t bb = __ballot(!ok);
      if (bb) {  // rare: a key without a valid slot
#pragma unroll
        for (int q = 0; q < RPI; q++) bad |= (uint32_t)((bb >> (q * CPR)) & 1u) << (i * RPI + q);
      }
      slot = ok ? slot : 0;
      // pool row of (slot, head h): page, head, position in page
      const uint32_t prow = (uint32_t)(slot >> 4) * (uint32_t)(a.Hkv * 16) + (uint32_t)(h * 16 + (slot & 15));
      const int pos = ln % CPR;
      const uint32_t dst = (uint32_t)(wave * IPW + i) * 1024u;
      const bf16_t* kp = a.k_pool + (size_t)prow * HD;
      const bf16_t* vp = a.v_pool + (size_t)prow * HD;
      dma16(kp + ((pos ^ Gm::swz_k(row)) * 8), __builtin_amdgcn_readfirstlane(lds_addr(kb + dst)));
      dma16(vp + ((pos ^ Gm::swz_v(row)) * 8), __builtin_amdgcn_readfirstlane(lds_addr(vb + dst)));
    }
    if (lane == 0) s_inval[st][wave] = (uint8_t)bad;
  };

  // Issue order keeps vmcnt accounting fixed: ... D(X), S(X+2), D(X+1) are the
  // last loads outstanding when tile X is waited for.
  if (nt > 0) {
    issue_slots(0);
    if (nt > 1) {
      issue_slots(1);
      wait_vmcnt<1>();
    } else {
      wait_vmcnt<0>();
    }
    issue_kv(0);
    if (nt > 1) {
      if (nt > 2) {
        issue_slots(2);
        wait_vmcnt<2 * IPW + 1>();
      } else {
        wait_vmcnt<2 * IPW>();
      }
      issue_kv(1);
    }
  }

  // tile X in ring stage ST (a constant, so every LDS read is a lane base
  // plus an immediate offset)
  auto tile = [&](int X, auto stc) {
    constexpr int st = decltype(stc)::value;
    if (X + 1 < nt) wait_vmcnt<2 * IPW>();
    else wait_vmcnt<0>();
    lds_barrier();  // stage X published; every wave is done with stage X - 1

    const uint8_t* kbs = s_kv + st * TILE;
    const uint8_t* vbs = s_kv + st * TILE;  // plus voff, which holds the V region base
    const int j0 = kbase + X * AKT;
    const uint64_t inval = *reinterpret_cast<const uint64_t*>(&s_inval[st][0]);
    const bool need_mask = (j0 + AKT - 1 > pmin) || (j0 < lomax) || inval != 0;

#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      // S^T: keys j0 + 32 kt + 8 (r / 4) + 4 g2 + r % 4, query column l32
      f32x16_t sacc = (f32x16_t){};
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const bf16x8_t kf =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kbs + kt * 32 * ROWB + koff[ks]));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc, 0, 0, 0);
      }
      if (kt == 0) {
        if (X + 3 < nt) issue_slots(X + 3);
        if (X + 2 < nt) issue_kv(X + 2);
      }
      // this half's V^T fragments, read now so the LDS latency hides under the softmax
      uint2 vr[2][DT][2];
#pragma unroll
      for (int cc = 0; cc < 2; cc++)
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
          vr[cc][dt][0] = lds_read_tr16(vbs + (16 * (2 * kt + cc)) * ROWB + voff[dt]);
          vr[cc][dt][1] = lds_read_tr16(vbs + (16 * (2 * kt + cc) + 8) * ROWB + voff[dt]);
        }
      __builtin_amdgcn_sched_barrier(0);
      // softmax over the query's 32 keys of this half: 16 here, 16 in lane ^ 32
      float sv[16];
#pragma unroll
      for (int r = 0; r < 16; r++) sv[r] = sacc[r];
      if (need_mask) {
        // register r holds key j0 + 32 kt + 4 g2 + kk, kk = 8 (r / 4) + r % 4:
        // outside [qlo, qpos], or bit kk of iv set (no valid slot), it is
        // excluded; the tests are selects, not branches
        const int kb = j0 + 32 * kt + 4 * g2;
        const int dq = qpos - kb, dl = qlo - kb;
        const uint32_t iv = (uint32_t)(inval >> (kt * 32 + 4 * g2));
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int kk = 8 * (r >> 2) + (r & 3);
          const bool bad = (kk > dq) | (kk < dl) | (((iv >> kk) & 1u) != 0u);
          sv[r] = bad ? -INFINITY : sv[r];
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int r = 1; r < 16; r++) mx = fmaxf(mx, sv[r]);
      mx = max_xor32(mx);
      const float mxs = mx * a.scale_log2;
      const bool grow = mxs > moff + 8.f;
      const float corr = grow ? __builtin_amdgcn_exp2f(moff - mxs) : 1.f;
      if (grow) moff = mxs;
      if (__any(grow)) {
        // (a splat-vector product: the scalar form trips a backend crash in this toolchain)
        const f32x16_t cv = {corr, corr, corr, corr, corr, corr, corr, corr,
                             corr, corr, corr, corr, corr, corr, corr, corr};
#pragma unroll
        for (int dt = 0; dt < DT; dt++) oacc[dt] = oacc[dt] * cv;
      }
      const float sub = moff == -INFINITY ? 0.f : moff;  // all scores -inf so far: p = 0
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        sv[r] = __builtin_amdgcn_exp2f(fmaf(sv[r], a.scale_log2, -sub));
        ls += sv[r];
      }
      lrow = lrow * corr + ls;
      // k step c = 2 kt + cc covers keys 16 c .. 16 c + 15: registers r = 8 cc .. 8 cc + 7
      uint4 pf[2];
#pragma unroll
      for (int cc = 0; cc < 2; cc++)
        pf[cc] = make_uint4(pack2_bf16(sv[8 * cc + 0], sv[8 * cc + 1]), pack2_bf16(sv[8 * cc + 2], sv[8 * cc + 3]),
                            pack2_bf16(sv[8 * cc + 4], sv[8 * cc + 5]), pack2_bf16(sv[8 * cc + 6], sv[8 * cc + 7]));
      // O^T[dt] += V^T[dims 32 dt .. +31][keys of step c] P^T: lane l supplies, for its
      // dim 32 dt + l % 32, keys 16 c + 4 g2 + 0..3 (u = 0) and 16 c + 8 + 4 g2 + 0..3 (u = 1)
#pragma unroll
      for (int cc = 0; cc < 2; cc++) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
          const uint2 v0 = vr[cc][dt][0], v1 = vr[cc][dt][1];
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8_t, pf[cc]), oacc[dt],
                                                             0, 0, 0);
        }
      }
    }
  };
  for (int X0 = 0; X0 < nt; X0 += ANST) {
    tile(X0, std::integral_constant<int, 0>{});
    if (X0 + 1 < nt) tile(X0 + 1, std::integral_constant<int, 1>{});
    if (X0 + 2 < nt) tile(X0 + 2, std::integral_constant<int, 2>{});
  }
  wait_vmcnt<0>();

  // oacc[dt][r] = O[query l32][dim dt*32 + 8 (r / 4) + 4 g2 + r % 4]
  float l = lrow;
  l += __shfl_xor(l, 32, 64);
  if (!qvalid) return;
  const int m = wave * 32 + l32;
  const int r = r0 + m / G, hq = h * G + m % G;
  if (a.n_split == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16_t* op = a.o + ((size_t)r * a.Hq + hq) * HD;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const f32x16_t x = oacc[dt];
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
        const f32x16_t x = oacc[dt];
        *reinterpret_cast<float4*>(op + dt * 32 + 8 * q4 + 4 * g2) =
            make_float4(x[q4 * 4 + 0], x[q4 * 4 + 1], x[q4 * 4 + 2], x[q4 * 4 + 3]);
      }
    if (g2 == 0) {
      a.part_ml[row * 2 + 0] = moff;
      a.part_ml[row * 2 + 1] = l;
    }
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

// ------------------------------------------------------------ few query rows
// One block per (row, KV head, key split), RW waves, each wave taking whole
// 64-key tiles of the split in turn; every query head of the GQA group rides
// along.  For a handful of rows (decode: one token per request) this reads
// each row's K/V once instead of running 256-row query blocks that are almost
// empty.  Per 64-key tile:
//   S^T = K Q^T    v_mfma_f32_16x16x32_bf16 on four 16-key subtiles, K rows
//                  loaded straight from the pool (lane l: key l % 16, dims
//                  8 (l / 16) + 32 ks .. + 7); query column c = head c of the
//                  group (columns >= G are zero);
//   softmax        per head, base 2, exact running maximum; probabilities go
//                  to the wave's LDS scratch, one row of 16 columns per key;
//   O += P V       on the vector units: lane l owns dims 8 (l % LPK) .. + 7 of
//                  every head for keys KPI i + l / LPK, V rows loaded straight
//                  from the pool; at the end the key groups are summed.
// The waves' (offset, sum, O) are combined in LDS and written as one split's
// partial (or, with one split, normalised to the output).
constexpr int RW = 4;  // waves per block
// one decode row over 8K keys, Mistral shape: 24 splits ran the decode step
// 0.5-1.5 % faster than 32, 16 and 48 (fewer partials to merge; some waves
// take two tiles)
constexpr int ROWS_SPLIT_MAX = 24;

template <int HD, int G>
__global__ void __launch_bounds__(64 * RW) attn_rows_kernel(AttnArgs a) {
  static_assert(G >= 1 && G <= 16, "group fits the 16 query columns");
  constexpr int KS = HD / 32;    // k32 steps over the head dim
  constexpr int LPK = HD / 8;    // lanes per key row in the V layout
  constexpr int KPI = 64 / LPK;  // keys per V load instruction
  constexpr int NI = 64 / KPI;   // V loads per 64-key tile
  __shared__ float s_p[RW][64][16];       // probabilities of the wave's tile: [key][query column]
  __shared__ float s_corr[RW][16];        // the tile's rescale factor per head
  __shared__ float s_o[RW][G][HD];        // per-wave results, combined at the end
  __shared__ float s_ml[RW][G][2];

  const int L = blockIdx.x;
  const int split = L % a.n_split, h = (L / a.n_split) % a.Hkv, r = L / (a.n_split * a.Hkv);
  const int M = row_count(a.n_rows, a.T_max);
  if (r >= M) return;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qc = lane & 15, kq = lane >> 4;     // S layout: query column, key quarter
  const int vj = lane % LPK, vg = lane / LPK;   // V layout: dim chunk, key group

  const int g = a.row_tok ? a.row_tok[r] : r;  // the row's token: keys tok_lo[g] .. g
  const int lo = a.tok_lo[g];
  const int ntiles = (g - lo) / 64 + 1;
  const int tb = (int)((long)ntiles * split / a.n_split), te = (int)((long)ntiles * (split + 1) / a.n_split);

  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qc < G) v = *reinterpret_cast<const uint4*>(a.q + ((size_t)r * a.Hq + h * G + qc) * HD + 32 * ks + 8 * kq);
    qf[ks] = __builtin_bit_cast(bf16x8_t, v);
  }

  float m_run = -INFINITY;  // running offset (base 2) of head qc, same in the 4 lanes of a column
  float l_run = 0.f;        // this lane's share of head qc's sum
  float oacc[G][8];
#pragma unroll
  for (int c = 0; c < G; c++)
#pragma unroll
    for (int e = 0; e < 8; e++) oacc[c][e] = 0.f;

  for (int T = tb + wave; T < te; T += RW) {
    const int k0 = lo + T * 64;
    // slot of key k0 + lane; keys past the row's token or without a valid slot are masked
    const int key = k0 + lane;
    int slot = key <= g ? a.slot_map[key] : -1;
    const bool ok = (unsigned)slot < (unsigned)a.n_slots;
    const uint64_t valid = __ballot(ok);
    slot = ok ? slot : 0;
    auto prow = [&](int sl) {
      return (size_t)((uint32_t)(sl >> 4) * (uint32_t)(a.Hkv * 16) + (uint32_t)(h * 16 + (sl & 15))) * HD;
    };
    // K fragments of the four 16-key subtiles, V rows of the lane's keys
    uint4 kr[4][KS], vr[NI];
#pragma unroll
    for (int qq = 0; qq < 4; qq++) {
      const size_t base = prow(__shfl(slot, 16 * qq + qc, 64)) + 8 * kq;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) kr[qq][ks] = *reinterpret_cast<const uint4*>(a.k_pool + base + 32 * ks);
    }
#pragma unroll
    for (int i = 0; i < NI; i++)
      vr[i] = *reinterpret_cast<const uint4*>(a.v_pool + prow(__shfl(slot, KPI * i + vg, 64)) + 8 * vj);

    // scores: sacc[qq][e] = S[key 16 qq + 4 kq + e][column qc]
    f32x4_t sacc[4];
#pragma unroll
    for (int qq = 0; qq < 4; qq++) {
      sacc[qq] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        sacc[qq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[qq][ks]), qf[ks],
                                                            sacc[qq], 0, 0, 0);
    }
    float sv[16];
    float mx = -INFINITY;
#pragma unroll
    for (int qq = 0; qq < 4; qq++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int kk = 16 * qq + 4 * kq + e;
        const bool in = (valid >> kk) & 1u;
        sv[4 * qq + e] = in ? sacc[qq][e] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[4 * qq + e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float corr = m_run == -INFINITY ? (m_new == -INFINITY ? 1.f : 0.f) : exp2f(m_run - m_new);
    m_run = m_new;
    const float sub = m_new == -INFINITY ? 0.f : m_new;
    float ls = 0.f;
#pragma unroll
    for (int qq = 0; qq < 4; qq++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float p = exp2f(sv[4 * qq + e] - sub);  // exp2(-inf) = 0 for masked keys
        ls += p;
        s_p[wave][16 * qq + 4 * kq + e][qc] = p;
      }
    l_run = l_run * corr + ls;
    if (kq == 0) s_corr[wave][qc] = corr;
    // (the wave's own LDS writes are read back in order: no barrier needed)
    float cf[G];
#pragma unroll
    for (int c = 0; c < G; c++) cf[c] = s_corr[wave][c];
#pragma unroll
    for (int c = 0; c < G; c++)
#pragma unroll
      for (int e = 0; e < 8; e++) oacc[c][e] *= cf[c];
#pragma unroll
    for (int i = 0; i < NI; i++) {
      float v8[8];
      unpack8_bf16(vr[i], v8);
      const float* pk = &s_p[wave][KPI * i + vg][0];
#pragma unroll
      for (int c = 0; c < G; c++) {
        const float p = pk[c];
#pragma unroll
        for (int e = 0; e < 8; e++) oacc[c][e] = fmaf(p, v8[e], oacc[c][e]);
      }
    }
  }

  // sum the key groups: lanes with the same dim chunk
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1)
#pragma unroll
    for (int c = 0; c < G; c++)
#pragma unroll
      for (int e = 0; e < 8; e++) oacc[c][e] += __shfl_xor(oacc[c][e], off, 64);
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (lane < LPK) {
#pragma unroll
    for (int c = 0; c < G; c++)
#pragma unroll
      for (int e = 0; e < 8; e++) s_o[wave][c][8 * vj + e] = oacc[c][e];
  }
  if (lane < G) {
    s_ml[wave][lane][0] = m_run;
    s_ml[wave][lane][1] = l_run;
  }
  __syncthreads();
  // combine the waves: thread (c, d) for head c, dim d
  for (int idx = t; idx < G * HD; idx += 64 * RW) {
    const int c = idx / HD, d = idx % HD;
    float mb = -INFINITY;
#pragma unroll
    for (int w = 0; w < RW; w++) mb = fmaxf(mb, s_ml[w][c][0]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < RW; w++) {
      const float mw = s_ml[w][c][0];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - mb);
      lsum += f * s_ml[w][c][1];
      osum += f * s_o[w][c][d];
    }
    const int hq = h * G + c;
    if (a.n_split == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      a.o[((size_t)r * a.Hq + hq) * HD + d] = (bf16_t)(pack2_bf16(osum * inv, 0.f) & 0xffffu);
    } else {
      const size_t row = ((size_t)split * a.T_max + r) * a.Hq + hq;
      a.part_o[row * HD + d] = osum;
      if (d == 0) {
        a.part_ml[row * 2 + 0] = mb;
        a.part_ml[row * 2 + 1] = lsum;
      }
    }
  }
}

// merge of split-KV partials: one wave per (row, head); base-2 exponents.
// Lane s reads split s's (offset, sum) once; the weighted sums then run over
// the splits in order with each weight broadcast from its lane, so the loads
// of different splits are independent (no chain of dependent loads per split).
template <int HD>
__global__ void __launch_bounds__(256) attn_merge_kernel(int T_max, const int32_t* __restrict__ n_rows, int Hq,
                                                         int n_split, const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, bf16_t* __restrict__ o) {
  const int w = (blockIdx.x * blockDim.x + threadIdx.x) >> 6, lane = threadIdx.x & 63;
  const int M = row_count(n_rows, T_max);
  if (w >= M * Hq) return;
  const size_t stride = (size_t)T_max * Hq;  // rows of one split
  float mx = -INFINITY;
  float acc[HD / 64] = {};
  float l = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += 64) {
    const int s = s0 + lane;
    const float ms = s < n_split ? part_ml[(s * stride + w) * 2] : -INFINITY;
    mx = fmaxf(mx, ms);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  for (int s0 = 0; s0 < n_split; s0 += 64) {
    const int sl = s0 + lane;
    float f = 0.f, ls = 0.f;
    if (sl < n_split) {
      const float ms = part_ml[(sl * stride + w) * 2];
      ls = part_ml[(sl * stride + w) * 2 + 1];
      f = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
    }
    const int ns = min(64, n_split - s0);
#pragma unroll 8
    for (int j = 0; j < ns; j++) {
      const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
      const float lj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), j));
      const size_t row = (size_t)(s0 + j) * stride + w;
      l += lj * fj;
#pragma unroll
      for (int e = 0; e < HD / 64; e++) acc[e] += fj * part_o[row * HD + lane + 64 * e];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < HD / 64; e++)
    o[(size_t)w * HD + lane + 64 * e] = (bf16_t)(pack2_bf16(acc[e] * inv, 0.f) & 0xffffu);
}

// The same merge with one 256-thread block per (row, head), for many splits
// and few rows: every split's partial is loaded at once (one memory round
// trip, staged in LDS), then thread d runs the merge of dim d with the
// arithmetic and order of attn_merge_kernel, so the output is bitwise the same.
constexpr int MERGE_WIDE_MAX = 64;
template <int HD>
__global__ void __launch_bounds__(256) attn_merge_wide_kernel(int T_max, const int32_t* __restrict__ n_rows, int Hq,
                                                              int n_split, const float* __restrict__ part_o,
                                                              const float* __restrict__ part_ml,
                                                              bf16_t* __restrict__ o) {
  __shared__ float s_o[MERGE_WIDE_MAX][HD];
  __shared__ float s_ml[MERGE_WIDE_MAX][2];
  const int w = blockIdx.x, t = threadIdx.x;  // w: (row, head)
  const int M = row_count(n_rows, T_max);
  if (w >= M * Hq) return;
  const size_t stride = (size_t)T_max * Hq;
  for (int i = t; i < n_split * 2; i += 256) s_ml[i >> 1][i & 1] = part_ml[((i >> 1) * stride + w) * 2 + (i & 1)];
  for (int i = t; i < n_split * (HD / 4); i += 256) {
    const int sp = i / (HD / 4), c = i % (HD / 4);
    *reinterpret_cast<float4*>(&s_o[sp][4 * c]) = *reinterpret_cast<const float4*>(part_o + (sp * stride + w) * HD + 4 * c);
  }
  __syncthreads();
  if (t >= HD) return;
  float mx = -INFINITY;
  for (int sp = 0; sp < n_split; sp++) mx = fmaxf(mx, s_ml[sp][0]);
  float l = 0.f, acc = 0.f;
  for (int sp = 0; sp < n_split; sp++) {
    const float ms = s_ml[sp][0], ls = s_ml[sp][1];
    const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
    l += ls * f;
    acc += f * s_o[sp][t];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  o[(size_t)w * HD + t] = (bf16_t)(pack2_bf16(acc * inv, 0.f) & 0xffffu);
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
    float s = -INFINITY;  // past the row's position, or no valid slot: excluded
    int slot = -1;
    if (j <= g) {
      slot = slot_map[j];
      if (slot >= 0 && slot < n_slots) {
        const float* kp = k_pool + kv_off(slot, h, Hkv, HD);
        float dot = 0.f;
        for (int i = 0; i < HD; i++) dot = fmaf(sq[i], kp[i], dot);
        s = dot * scale;
      }
    }
    const float mx = wave_max(s);
    const float mnew = fmaxf(m, mx);
    const float corr = mnew == -INFINITY ? 1.f : expf(m - mnew);
    const float p = s == -INFINITY ? 0.f : expf(s - mnew);
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
// rows up to this count use the few-rows kernel (bf16, group of 1..16 heads)
constexpr int ROWS_MAX = 4;
static bool rows_kernel_ok(const kvb_model_desc* d, int T_max) {
  const int G = d->n_q_heads / d->n_kv_heads;
  return T_max <= ROWS_MAX && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16) &&
         (d->head_dim == 64 || d->head_dim == 128);
}

int attn_splits(const kvb_model_desc* d, int T_max, int n_cu) {
  if (rows_kernel_ok(d, T_max)) {
    // every (row, KV head, split) block 4 waves; about two blocks per CU
    const long items = (long)T_max * d->n_kv_heads;
    const long s = (2L * n_cu + items - 1) / items;
    return (int)(s < 1 ? 1 : (s > ROWS_SPLIT_MAX ? ROWS_SPLIT_MAX : s));
  }
  // about 1.2 work items per CU: measured best at 334, 819, 992, 1300, 2129
  // and 8192 rows of the Mistral shape (more splits add partial traffic and
  // merge work faster than they even out the causal item lengths)
  const int G = d->n_q_heads / d->n_kv_heads;
  const long items = (long)cdiv(T_max, AQ / G) * d->n_kv_heads;
  const long s = (6L * n_cu + 5 * items - 1) / (5 * items);
  return (int)(s < 1 ? 1 : (s > 16 ? 16 : s));
}

size_t ws_attn_bytes(const kvb_model_desc* d, int32_t max_rows, int n_cu) {
  if (d->dtype != KVB_BF16) return 0;
  // largest n_split * T over T <= max_rows (n_split shrinks as T grows)
  size_t best = 0;
  const int G = d->n_q_heads / d->n_kv_heads, TB = AQ / G;
  for (int T = 1; T <= ROWS_MAX && T <= max_rows; T++) best = std::max(best, (size_t)attn_splits(d, T, n_cu) * T);
  for (int qb = 1; qb <= cdiv(max_rows, TB); qb++) {
    const int T = qb * TB < max_rows ? qb * TB : max_rows;
    const int s = attn_splits(d, T, n_cu);
    if (s == 1) break;
    best = std::max(best, (size_t)s * T);
  }
  if (best == 0) return 0;
  return align_up(best * d->n_q_heads * d->head_dim * 4, 256) + align_up(best * d->n_q_heads * 2 * 4, 256);
}

static kvb_status launch_merge(hipStream_t st, int hd, int T_max, const int32_t* n_rows, int Hq, int n_split,
                               const float* part_o, const float* part_ml, bf16_t* o) {
  {
    LaunchTimer lt(st, "attention_merge");
    const int waves = T_max * Hq;
    if (n_split >= 8 && n_split <= MERGE_WIDE_MAX && waves <= 4096) {
      if (hd == 128) attn_merge_wide_kernel<128><<<waves, 256, 0, st>>>(T_max, n_rows, Hq, n_split, part_o, part_ml, o);
      else attn_merge_wide_kernel<64><<<waves, 256, 0, st>>>(T_max, n_rows, Hq, n_split, part_o, part_ml, o);
    } else if (hd == 128)
      attn_merge_kernel<128><<<cdiv(waves, 4), 256, 0, st>>>(T_max, n_rows, Hq, n_split, part_o, part_ml, o);
    else
      attn_merge_kernel<64><<<cdiv(waves, 4), 256, 0, st>>>(T_max, n_rows, Hq, n_split, part_o, part_ml, o);
  }
  return check_launch("attn_merge_kernel");
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
  if ((long)n_pages * desc->n_kv_heads * 16 > 0xffffffffL)
    return fail(KVB_ERR_UNSUPPORTED, "pool rows (pages x KV heads x 16) must fit 32 bits");
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
    if (rows_kernel_ok(desc, T_max)) {
      // a handful of rows: one block per (row, KV head, split)
      const dim3 rgrid((unsigned)((long)T_max * Hkv * n_split));
      {
        LaunchTimer lt(st, "attention");
        if (hd == 128) {
          switch (G) {
            case 1: attn_rows_kernel<128, 1><<<rgrid, 64 * RW, 0, st>>>(a); break;
            case 2: attn_rows_kernel<128, 2><<<rgrid, 64 * RW, 0, st>>>(a); break;
            case 4: attn_rows_kernel<128, 4><<<rgrid, 64 * RW, 0, st>>>(a); break;
            case 8: attn_rows_kernel<128, 8><<<rgrid, 64 * RW, 0, st>>>(a); break;
            default: attn_rows_kernel<128, 16><<<rgrid, 64 * RW, 0, st>>>(a); break;
          }
        } else {
          switch (G) {
            case 1: attn_rows_kernel<64, 1><<<rgrid, 64 * RW, 0, st>>>(a); break;
            case 2: attn_rows_kernel<64, 2><<<rgrid, 64 * RW, 0, st>>>(a); break;
            case 4: attn_rows_kernel<64, 4><<<rgrid, 64 * RW, 0, st>>>(a); break;
            case 8: attn_rows_kernel<64, 8><<<rgrid, 64 * RW, 0, st>>>(a); break;
            default: attn_rows_kernel<64, 16><<<rgrid, 64 * RW, 0, st>>>(a); break;
          }
        }
      }
      KVB_TRY(check_launch("attn_rows_kernel"));
      if (n_split > 1) KVB_TRY(launch_merge(st, hd, T_max, n_rows, Hq, n_split, a.part_o, a.part_ml, (bf16_t*)o));
      return KVB_OK;
    }
    // one block per (query block, KV head, split) item, in the XCD order the kernel decodes
    const long per_head = (long)a.n_qblocks * n_split;
    long blocks = per_head * Hkv;
    if (Hkv % 8 != 0 && 8 % Hkv == 0) blocks = 8L * ((per_head + 8 / Hkv - 1) / (8 / Hkv));
    if (blocks > 0x7fffffffL) return fail(KVB_ERR_UNSUPPORTED, "attention grid too large");
    const dim3 grid((unsigned)blocks);
    {
      LaunchTimer lt(st, "attention", true);
      if (hd == 128)
        hipExtLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(ATHREADS), 0, st, lt.start(), lt.stop(), 0, a);
      else
        hipExtLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(ATHREADS), 0, st, lt.start(), lt.stop(), 0, a);
    }
    KVB_TRY(check_launch("attn_bf16_kernel"));
    if (n_split > 1) KVB_TRY(launch_merge(st, hd, T_max, n_rows, Hq, n_split, a.part_o, a.part_ml, (bf16_t*)o));
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
