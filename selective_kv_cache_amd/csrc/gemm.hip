// Gathered-row GEMMs of the link step: the Q/K/V projection and the output
// projection + SwiGLU MLP of the recomputed rows (EPIC page, section 4,
// LegoLink steps 2 and 5; the same per-layer dataflow serves CacheSlide).
//
//   C[m, n] = sum_k A[row(m), k] * W[n, k]      (W is [N, K], row-major)
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 on gfx950 (see the bf16 section).
// fp32 path: an LDS-tiled FMA kernel with the same epilogues (used by the
// small float32 workload), RMSNorm folded into its A loads.
//
// Fusions: epilogues split Q/K/V, add the residual, apply SiLU(gate) * up on a
// dual-B tile, or scatter rows back to the hidden buffer.  For bf16, RMSNorm
// runs as a row pre-pass (rmsnorm_rows_kernel) whose bf16 output the
// projection reads.
//
// Row invariance: for the Q/K/V projection the reduction order of every output
// element (K stages in order, the MFMA's k slices in order) and of every
// row's sum of squares depends only on k, never on the row's index or on M,
// so a row's result is the same whatever batch it is computed in.  The MLP
// products may split K across blocks (stream-K); their results are
// deterministic for a given batch.
#include "common.h"

#include <algorithm>
#include <functional>
#include <vector>
#include <type_traits>

namespace kvb {

enum EpiMode { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_SCATTER = 3 };

template <class T>
struct GemmArgs {
  const T* A;                 // [*, K] rows
  const int32_t* a_rows;      // gather (nullptr: identity)
  const T* B;                 // [N, K]
  const T* B2;                // dual-B second matrix [N, K] (SwiGLU up rows)
  const T* norm_w;            // RMSNorm gains [K] (nullptr: no norm)
  int M_max;
  const int32_t* n_rows;      // device row count (nullptr: M_max)
  int N, K;
  float eps;
  // epilogue
  T* out0;
  T* out1;
  T* out2;
  int n0, n1;                 // Q|K|V split points
  int ldo;
  const T* resid;
  const int32_t* resid_rows;
  int ldr;
  const int32_t* out_rows;
};

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }
// bf16 epilogues: the hardware reciprocal (about 1 ulp) instead of an IEEE
// division; the result is rounded to bf16 right after
__device__ __forceinline__ float silu_bf16(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

template <int MODE, class T>
__device__ __forceinline__ void epilogue(const GemmArgs<T>& p, int m, int n, float acc, float acc2, float rinv) {
  if (MODE == EPI_QKV) {
    const float v = acc * rinv;
    if (n < p.n0) Store<T>::st(p.out0 + (size_t)m * p.n0 + n, v);
    else if (n < p.n1) Store<T>::st(p.out1 + (size_t)m * (p.n1 - p.n0) + (n - p.n0), v);
    else Store<T>::st(p.out2 + (size_t)m * (p.N - p.n1) + (n - p.n1), v);
  } else if (MODE == EPI_RESID) {
    const int rr = p.resid_rows ? p.resid_rows[m] : m;
    const float h = to_f<T>(p.resid[(size_t)rr * p.ldr + n]);
    Store<T>::st(p.out0 + (size_t)m * p.ldo + n, h + acc);
  } else if (MODE == EPI_SWIGLU) {
    Store<T>::st(p.out0 + (size_t)m * p.ldo + n, silu(acc * rinv) * (acc2 * rinv));
  } else {  // EPI_SCATTER
    const int orow = p.out_rows ? p.out_rows[m] : m;
    const float h = to_f<T>(p.resid[(size_t)m * p.ldr + n]);
    Store<T>::st(p.out0 + (size_t)orow * p.ldo + n, h + acc);
  }
}

// ====================================================================== bf16 MFMA
//
// Block = 8 waves in a WM x WN grid (two waves per SIMD, at most 256 registers
// each, so one wave's MFMAs run while the other waits on LDS or a barrier);
// wave tile = (32 TM) x (32 TN) outputs as TM x TN tiles of
// v_mfma_f32_32x32x16_bf16; block tile BM x BN.  K advances KB (32 or 64) per
// stage through a ring of NST LDS stages filled by direct-to-LDS loads
// (global_load_lds_dwordx4 with a scalar base and 32-bit lane offsets).  With
// three or more stages the next stage is published one step ahead, so the
// first MFMA fragments of a stage are read while the previous stage computes;
// inside a stage the fragments of the next k16 step are read while the
// current step's MFMAs run.
//
// LDS stage layout: rows of 2 KB bytes; the 16-byte chunk c of row r is stored
// at position c ^ swizzle(r), which makes the fragment reads of 16 consecutive
// rows hit 16 distinct bank groups.  A wave's load instruction fills 1 KiB =
// RPI rows; its lane j fetches row j / CPR, chunk (j % CPR) ^ swizzle(row).
//
// SwiGLU (DUAL): the B tile interleaves 32-row subtiles of the gate and up
// matrices (gate cols c..c+31, up cols c..c+31, ...), so a wave holds gate
// and up of the same outputs in neighbouring accumulators; BN/2 outputs wide.
//
// Split-K (SK): when whole tiles would fill the chip unevenly, each tile's K
// steps are cut into S slices run by S blocks, each writing its float partial
// [S][rows][cols]; splitk_reduce_kernel then adds the S partials in slice
// order and applies the epilogue.  The reduction order depends on the launch,
// so split-K is used only for the MLP products, never for the Q/K/V
// projection (whose per-row results must not depend on the batch).
//
// RMSNorm is not fused here: rmsnorm_rows_kernel writes the normalised rows
// (bf16, one rounding) to workspace and the GEMM reads them as a plain A.

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ void unpack8(const uint4& a, float (&f)[8]) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// y[r] = x[a_rows[r]] * rinv_r * g (bf16, one rounding), rinv_r =
// 1 / sqrt(mean(x^2) + eps), for r < *n_rows; g == NULL means unit gains.
// One wave per row: lane l sums the 16-byte chunks l, l + 64, ... in order,
// then a fixed butterfly; the result depends on the row's values only.
__global__ void __launch_bounds__(256) rmsnorm_rows_kernel(const bf16_t* __restrict__ x,
                                                           const int32_t* __restrict__ a_rows,
                                                           const int32_t* __restrict__ n_rows, int T_max, int K,
                                                           const bf16_t* __restrict__ g, float eps,
                                                           bf16_t* __restrict__ y) {
  const int r = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= row_count(n_rows, T_max)) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)(a_rows ? a_rows[r] : r) * K);
  uint4* yr = reinterpret_cast<uint4*>(y + (size_t)r * K);
  const int C = K / 8;
  float s = 0.f;
  for (int c = lane; c < C; c += 64) {
    float f[8];
    unpack8(xr[c], f);
#pragma unroll
    for (int e = 0; e < 8; e++) s += f[e] * f[e];
  }
  s = wave_sum(s);
  const float rinv = 1.f / sqrtf(s / (float)K + eps);
  for (int c = lane; c < C; c += 64) {
    float f[8], w[8];
    unpack8(xr[c], f);
    if (g) unpack8(reinterpret_cast<const uint4*>(g)[c], w);
#pragma unroll
    for (int e = 0; e < 8; e++) f[e] = g ? f[e] * rinv * w[e] : f[e] * rinv;
    yr[c] = make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]), pack2_bf16(f[6], f[7]));
  }
}

// The same arithmetic in the same order for K = 512 CPL: the whole row (and
// the gains) is loaded into registers up front, so the row costs one memory
// latency instead of one per chunk.
template <int CPL>
__global__ void __launch_bounds__(256) rmsnorm_rows_reg_kernel(const bf16_t* __restrict__ x,
                                                               const int32_t* __restrict__ a_rows,
                                                               const int32_t* __restrict__ n_rows, int T_max,
                                                               const bf16_t* __restrict__ g, float eps,
                                                               bf16_t* __restrict__ y) {
  constexpr int K = 512 * CPL;
  const int r = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= row_count(n_rows, T_max)) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)(a_rows ? a_rows[r] : r) * K);
  uint4* yr = reinterpret_cast<uint4*>(y + (size_t)r * K);
  const uint4* gr = reinterpret_cast<const uint4*>(g);
  uint4 xv[CPL], gv[CPL];
#pragma unroll
  for (int i = 0; i < CPL; i++) xv[i] = xr[lane + 64 * i];
  if (g) {
#pragma unroll
    for (int i = 0; i < CPL; i++) gv[i] = gr[lane + 64 * i];
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; i++) {
    float f[8];
    unpack8(xv[i], f);
#pragma unroll
    for (int e = 0; e < 8; e++) s += f[e] * f[e];
  }
  s = wave_sum(s);
  const float rinv = 1.f / sqrtf(s / (float)K + eps);
#pragma unroll
  for (int i = 0; i < CPL; i++) {
    float f[8], w[8];
    unpack8(xv[i], f);
    if (g) unpack8(gv[i], w);
#pragma unroll
    for (int e = 0; e < 8; e++) f[e] = g ? f[e] * rinv * w[e] : f[e] * rinv;
    yr[lane + 64 * i] = make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]),
                                   pack2_bf16(f[6], f[7]));
  }
}

static kvb_status rmsnorm_rows(hipStream_t st, const bf16_t* x, const int32_t* a_rows, const int32_t* n_rows,
                               int T_max, int K, const bf16_t* g, float eps, bf16_t* y) {
  {
    LaunchTimer lt(st, "rmsnorm");
    const dim3 grid(cdiv(T_max, 4)), block(256);
    switch (K) {
      case 2048: rmsnorm_rows_reg_kernel<4><<<grid, block, 0, st>>>(x, a_rows, n_rows, T_max, g, eps, y); break;
      case 4096: rmsnorm_rows_reg_kernel<8><<<grid, block, 0, st>>>(x, a_rows, n_rows, T_max, g, eps, y); break;
      case 5120: rmsnorm_rows_reg_kernel<10><<<grid, block, 0, st>>>(x, a_rows, n_rows, T_max, g, eps, y); break;
      case 8192: rmsnorm_rows_reg_kernel<16><<<grid, block, 0, st>>>(x, a_rows, n_rows, T_max, g, eps, y); break;
      default: rmsnorm_rows_kernel<<<grid, block, 0, st>>>(x, a_rows, n_rows, T_max, K, g, eps, y);
    }
  }
  return check_launch("rmsnorm_rows_kernel");
}

constexpr int GEMM_WAVES = 8;
constexpr int GEMM_THREADS = 64 * GEMM_WAVES;

template <int BM_, int BN_, int WM_, int KB_, int NST_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = GEMM_WAVES / WM_, KB = KB_, NST = NST_;
  static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // MFMA tiles per wave
  static constexpr int ROWB = KB * 2;                          // bytes per tile row per stage
  static constexpr int CPR = ROWB / 16;                        // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                         // rows per 1 KiB load instruction
  static constexpr int A_I = BM / RPI / GEMM_WAVES, B_I = BN / RPI / GEMM_WAVES;  // loads per wave per stage
  static constexpr int PER = A_I + B_I;
  static constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static constexpr int KS = KB / 16;                           // k16 steps per stage
  static constexpr int EPI_BYTES = 32 * (BN + 8) * 4;          // one 32-row epilogue phase
  static constexpr int ARR = STAGE_BYTES > EPI_BYTES ? STAGE_BYTES : EPI_BYTES;
  static constexpr int NACC = TM * TN * 16;                    // accumulator floats per lane
  static_assert(TM >= 1 && TN >= 1 && A_I >= 1 && B_I >= 1 && NST >= 2, "tile shape");
  __device__ __forceinline__ static int swz(int r) { return KB == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
};

// The ring: NST stages of ARR bytes in one LDS object; the K loop is unrolled
// by NST, so every stage address is a compile-time constant.
template <class TL>
struct RingLds {
  __device__ static uint8_t* ptr() {
    __shared__ __align__(16) uint8_t buf[TL::NST * TL::ARR];
    return buf;
  }
};

// 16 bytes per lane from base + off (scalar base, 32-bit lane byte offset),
// landing at LDS address lds_base + 16 * lane
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds_base) : "memory");
}

// wait until at most `allowed` (a multiple of the per-stage load count, <= N)
// direct-to-LDS loads are outstanding
template <int N>
__device__ __forceinline__ void wait_vm_upto(int allowed) {
  if constexpr (N <= 0) {
    wait_vmcnt<0>();
  } else {
    if (allowed >= N) wait_vmcnt<N>();
    else wait_vm_upto<N - 1>(allowed);
  }
}

// split-K schedule of one launch
struct SkArgs {
  int S;           // K slices per tile (1: no split); a mixed plan gives a tile S or S + 1
  int rows;        // row stride of a slice: M_max rounded up to the tile height
  int cols;        // N (DUAL: 2 N, gate columns then up columns)
  float* part;     // [slice][rows][cols]
  // Mixed plan (xcd_blocks > 0): the tile order is cut into 8 contiguous runs,
  // run x for the blocks of XCD x; a run of n tiles gives its last
  // h = clamp(xcd_blocks - n S, 0, n) tiles S + 1 slices and the others S,
  // and its S-slice blocks come first, so whole rounds of blocks fill the CUs.
  int xcd_blocks;
  int bm, bn;      // tile rows and output columns; tiles per column and row
  int num_m, num_n;
};

// run x of a mixed plan: first tile t0, nt tiles, the last nh of them with S + 1 slices
__host__ __device__ inline void mixed_run(int tiles, int x, int S, int xcd_blocks, int& t0, int& nt, int& nh) {
  t0 = (int)((long)x * tiles / 8);
  nt = (int)((long)(x + 1) * tiles / 8) - t0;
  nh = xcd_blocks - nt * S;
  nh = nh < 0 ? 0 : (nh > nt ? nt : nh);
}

// grouped tile order: GM m-tiles sweep all n-tiles, so concurrent tiles share panels
__device__ __forceinline__ void tile_coords(int t, int num_m, int num_n, int& tm, int& tn) {
  const int GM = num_m <= 16 ? num_m : 8;
  const int gsize = GM * num_n;
  const int grp = t / gsize, first = grp * GM;
  const int gm = min(GM, num_m - first);
  const int in = t - grp * gsize;
  tm = first + in % gm;
  tn = in / gm;
}

// inverse of tile_coords
__device__ __forceinline__ int tile_index(int tm, int tn, int num_m, int num_n) {
  const int GM = num_m <= 16 ? num_m : 8;
  const int grp = tm / GM, first = grp * GM;
  const int gm = min(GM, num_m - first);
  return grp * GM * num_n + tn * gm + (tm - first);
}

// Epilogue staging of a tile with OUT_N output columns: float slabs of 32
// rows x (OUT_N + 8) (rows 4 apart land 32 banks apart), SPS of them in each
// ring stage; each phase fills G slabs per wave row, G the largest divisor of
// the wave's subtile count whose WM * G slabs fit the ring.
template <class TL, int OUT_N>
struct EpiPlan {
  static constexpr int SLAB = 32 * (OUT_N + 8) * 4;
  static constexpr int SPS = TL::ARR / SLAB;
  static constexpr int pick() {
    int g = TL::TM;
    while (g > 1 && (TL::TM % g || TL::WM * g > TL::NST * SPS)) g--;
    return g;
  }
  static constexpr int G = pick();
  static_assert(TL::WM * G <= TL::NST * SPS, "epilogue slabs exceed the ring");
  static_assert(TL::WM * G * 32 * (OUT_N / 8) % GEMM_THREADS == 0, "epilogue chunks per thread");
};

template <int MODE, bool DUAL, class TL, bool SK>
__global__ void __launch_bounds__(GEMM_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_bf16_kernel(GemmArgs<bf16_t> p, SkArgs sk) {
  constexpr int BM = TL::BM, BN = TL::BN, WN = TL::WN, TM = TL::TM, TN = TL::TN, KB = TL::KB, NST = TL::NST;
  constexpr int A_I = TL::A_I, B_I = TL::B_I, PER = TL::PER, ROWB = TL::ROWB, CPR = TL::CPR, RPI = TL::RPI;
  constexpr int KS = TL::KS;
  constexpr int OUT_N = DUAL ? BN / 2 : BN;  // output columns per block
  constexpr bool PA = NST >= 3;              // publish the next stage one step ahead
  static_assert(!DUAL || TN % 2 == 0, "SwiGLU pairs gate and up subtiles inside a wave");
  uint8_t* const ring = RingLds<TL>::ptr();
  uint8_t* const stg[4] = {ring, ring + TL::ARR, ring + 2 * TL::ARR, ring + 3 * TL::ARR};  // stages < NST

  const int M = row_count(p.n_rows, p.M_max);
  const int num_m = cdiv_dev(p.M_max, BM), num_n = cdiv_dev(p.N, OUT_N);
  const int tiles = num_m * num_n;
  const int KT = p.K / KB;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = (wave / WN) * (32 * TM), wn = (wave % WN) * (32 * TN);
  const int lrow = lane / CPR, lpos = lane % CPR;
  const int fr = lane & 31, fh = lane >> 5, fs = TL::swz(fr);
  const bf16_t* const Bup = DUAL ? p.B2 : p.B;

  // this block's work: K slice `split` of one tile.  Workgroups go to the 8
  // XCDs round-robin (id % 8), each XCD with its own L2: give every XCD a
  // contiguous run of the (tile, slice) order.
  int tile, split, S;
  if (SK && sk.xcd_blocks > 0) {
    int t0, nt, nh;
    mixed_run(tiles, (int)(blockIdx.x & 7), sk.S, sk.xcd_blocks, t0, nt, nh);
    const int li = (int)(blockIdx.x >> 3), n_long = (nt - nh) * sk.S;
    if (li >= n_long + nh * (sk.S + 1)) return;
    if (li < n_long) {
      S = sk.S;
      tile = t0 + li / S;
      split = li % S;
    } else {
      S = sk.S + 1;
      tile = t0 + (nt - nh) + (li - n_long) / S;
      split = (li - n_long) % S;
    }
  } else {
    S = SK ? sk.S : 1;
    const int total = tiles * S;
    const int per = (total + 7) >> 3;
    const int tid = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (tid >= total) return;
    tile = tid / S;
    split = tid - tile * S;
  }
  const int kbeg = split * KT / S, kend = (split + 1) * KT / S;
  {
    f32x16_t acc[TM][TN];
    uint4 fa[2][TM], fb[2][TN];
    int tm, tn;
    tile_coords(tile, num_m, num_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * OUT_N;
    // rows past the device row count: nothing to compute or store (every slice
    // of such a tile leaves here, so its counter is never touched)
    if (m0 >= M) return;
    const int KTL = kend - kbeg;

    // ---- direct-to-LDS loaders: instruction i of this wave covers tile rows
    //      (wave * X_I + i) * RPI + lane / CPR, lane position lane % CPR
    uint32_t a_off[A_I], b_off[B_I];
#pragma unroll
    for (int i = 0; i < A_I; i++) {
      const int r = (wave * A_I + i) * RPI + lrow;
      int m = m0 + r;
      m = m < M ? m : M - 1;
      m = m < 0 ? 0 : m;
      const int ar = p.a_rows ? p.a_rows[m] : m;
      a_off[i] = (uint32_t)(((size_t)ar * p.K + (size_t)((lpos ^ TL::swz(r)) * 8)) * 2);
    }
#pragma unroll
    for (int i = 0; i < B_I; i++) {
      const int r = (wave * B_I + i) * RPI + lrow;  // B-tile row; 32-row subtile r / 32
      int n;
      size_t base = 0;
      if (DUAL) {
        n = n0 + (r >> 6) * 32 + (r & 31);
        if ((r >> 5) & 1) base = (size_t)(Bup - p.B);
      } else {
        n = n0 + r;
      }
      n = n < p.N ? n : p.N - 1;
      b_off[i] = (uint32_t)((base + (size_t)n * p.K + (size_t)((lpos ^ TL::swz(r)) * 8)) * 2);
    }
    auto issue = [&](int j, uint8_t* st) {
      const size_t ko = (size_t)(kbeg + j) * KB;
      const bf16_t* ab = p.A + ko;
      const bf16_t* bb = p.B + ko;
#pragma unroll
      for (int i = 0; i < A_I; i++)
        dma16s(ab, a_off[i], __builtin_amdgcn_readfirstlane(lds_addr(st + (wave * A_I + i) * 1024)));
#pragma unroll
      for (int i = 0; i < B_I; i++)
        dma16s(bb, b_off[i], __builtin_amdgcn_readfirstlane(lds_addr(st + BM * ROWB + (wave * B_I + i) * 1024)));
    };
    auto frags = [&](int buf, const uint8_t* st, int s) {
      const int off = fr * ROWB + (((2 * s + fh) ^ fs) * 16);
#pragma unroll
      for (int i = 0; i < TM; i++) fa[buf][i] = *reinterpret_cast<const uint4*>(st + (wm + 32 * i) * ROWB + off);
#pragma unroll
      for (int j = 0; j < TN; j++)
        fb[buf][j] = *reinterpret_cast<const uint4*>(st + BM * ROWB + (wn + 32 * j) * ROWB + off);
    };
    auto mma = [&](int buf) {
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[buf][i]), as_bf16x8(fb[buf][j]), acc[i][j],
                                                              0, 0, 0);
    };

#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++) acc[i][j] = (f32x16_t){};

    // ---- K loop over [kbeg, kend)
#pragma unroll
    for (int j = 0; j < NST - 1; j++)
      if (j < KTL) issue(j, stg[j]);
    if constexpr (PA) {
      if (KTL > 0) {
        wait_vm_upto<(NST - 2) * PER>(min(KTL - 1, NST - 2) * PER);
        lds_barrier();
        frags(0, stg[0], 0);
      }
    }
    for (int kt0 = 0; kt0 < KTL; kt0 += NST) {
#pragma unroll
      for (int S = 0; S < NST; S++) {
        const int kt = kt0 + S;
        if (kt < KTL) {
          if constexpr (PA) wait_vm_upto<(NST - 3) * PER>(max(0, min(KTL - 2 - kt, NST - 3)) * PER);
          else wait_vmcnt<0>();
          lds_barrier();  // stage kt (PA: kt + 1) published; every wave is done with the stage refilled next
          if (kt + NST - 1 < KTL) issue(kt + NST - 1, stg[(S + NST - 1) % NST]);
          if constexpr (!PA) {
            frags(0, stg[S], 0);
            __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);  // this slice's reads come first
          }
#pragma unroll
          for (int s = 0; s < KS; s++) {
            if (s + 1 < KS) frags((s + 1) & 1, stg[S], s + 1);
            else if (PA && kt + 1 < KTL) frags((s + 1) & 1, stg[(S + 1) % NST], 0);
            mma(s & 1);
            if (s + 1 < KS) {
              // keep the next slice's fragment reads ahead of this slice's
              // MFMAs (left alone, the scheduler sinks each read to just
              // before its use and the MFMAs wait on LDS latency)
              __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);  // LDS reads
              __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);  // MFMAs
            }
          }
        }
      }
    }
    wait_vmcnt<0>();
    lds_barrier();  // every wave is done with the ring before the epilogue reuses LDS

    // ---- split-K: write this slice's partial (row-major, the reduction kernel
    // applies the epilogue)
    if constexpr (SK) {
      float* dst = sk.part + (size_t)split * sk.rows * sk.cols;
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) {
          // DUAL: subtile j even holds gate, odd holds up, of output cols (wn / 32 + j) / 2 * 32
          const int col = DUAL ? ((j & 1) ? p.N : 0) + n0 + ((wn / 32 + j) >> 1) * 32 + (lane & 31)
                               : n0 + wn + 32 * j + (lane & 31);
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row < M && (DUAL ? ((j & 1) ? col - p.N : col) : col) < p.N)
              dst[(size_t)row * sk.cols + col] = acc[i][j][r];
          }
        }
      return;
    }

    // ---- epilogue, staged through LDS: in each phase every wave row writes
    // the float accumulators (SwiGLU already combined) of G of its 32-row
    // subtiles to slabs [32][OUT_N + 8] in the ring's stages, then all threads
    // read 8 consecutive outputs of a row, apply the mode (residual, scatter)
    // and store 16 bytes at a time.  The gather / scatter indices and residual
    // rows of every chunk a thread stores are loaded before its first store,
    // so no wait for them also waits for a store (vmcnt counts both).
    // acc[i][j][r] sits at tile row wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,
    // tile col wn + 32 j + lane % 32 (DUAL: output col (wn / 32 + j) / 2 * 32 + lane % 32).
    using EP = EpiPlan<TL, OUT_N>;
    constexpr int G = EP::G, LDC = OUT_N + 8, CPRO = OUT_N / 8;
    constexpr int NPH = TM / G;                                 // phases
    constexpr int NCH = TL::WM * G * 32 * CPRO / GEMM_THREADS;  // chunks per thread per phase
    constexpr bool LOADS = MODE == EPI_RESID || MODE == EPI_SCATTER;
    const int wr = wave / WN, lc = lane & 31;
    // slab s = wave row * G + g: ring stage s % NST, slab (s / NST) of that stage
    auto slab = [&](int s) { return reinterpret_cast<float*>(ring + (s % NST) * TL::ARR + (s / NST) * EP::SLAB); };
    // thread t stores chunks k of each phase: phase row q = t / CPRO + k * (GEMM_THREADS / CPRO)
    // (slab q / 32, row q % 32), columns n0 + cc .. + 7
    const int cc = (t % CPRO) * 8, n = n0 + cc;
    auto tile_row = [&](int ph, int k) {
      const int q = t / CPRO + k * (GEMM_THREADS / CPRO), s = q >> 5;
      return (s / G) * 32 * TM + (ph * G + s % G) * 32 + (q & 31);
    };
    uint4 hres[LOADS ? NPH : 1][LOADS ? NCH : 1];
    int orow[MODE == EPI_SCATTER ? NPH : 1][MODE == EPI_SCATTER ? NCH : 1];
    if constexpr (LOADS) {
      // clamped into range, so every load is issued (invalid chunks store nothing)
      const int nl = n < p.N ? n : p.N - 8;
      const int32_t* gidx = MODE == EPI_RESID ? p.resid_rows : p.out_rows;
      int rr[NPH][NCH];
#pragma unroll
      for (int ph = 0; ph < NPH; ph++)
#pragma unroll
        for (int k = 0; k < NCH; k++) {
          const int m = min(m0 + tile_row(ph, k), M - 1);
          const int g = gidx ? gidx[m] : m;
          if constexpr (MODE == EPI_SCATTER) orow[ph][k] = g;
          rr[ph][k] = MODE == EPI_RESID ? g : m;
        }
#pragma unroll
      for (int ph = 0; ph < NPH; ph++)
#pragma unroll
        for (int k = 0; k < NCH; k++)
          hres[ph][k] = *reinterpret_cast<const uint4*>(p.resid + (size_t)rr[ph][k] * p.ldr + nl);
    }
#pragma unroll
    for (int ph = 0; ph < NPH; ph++) {
#pragma unroll
      for (int g = 0; g < G; g++) {
        const int i = ph * G + g;
        float* sC = slab(wr * G + g);
#pragma unroll
        for (int j = 0; j < TN; j += (DUAL ? 2 : 1)) {
          const int cl = DUAL ? ((wn / 32 + j) >> 1) * 32 + lc : wn + j * 32 + lc;
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);  // row inside the subtile
            float v = acc[i][j][r];
            if (DUAL) v = silu_bf16(v) * acc[i][j + 1][r];
            sC[rl * LDC + cl] = v;
          }
        }
      }
      lds_barrier();
      // the residual loads, issued before the first slab fill, are all in
      // before any store is issued (the stores sit in branches, which the
      // compiler's own wait counts cannot see past)
      if (LOADS && ph == 0) wait_vmcnt<0>();
#pragma unroll
      for (int k = 0; k < NCH; k++) {
        const int q = t / CPRO + k * (GEMM_THREADS / CPRO);
        const int m = m0 + tile_row(ph, k);
        if (m >= M || n >= p.N) continue;
        const float* src = slab(q >> 5) + (q & 31) * LDC + cc;
        const float4 lo = *reinterpret_cast<const float4*>(src);
        const float4 hi = *reinterpret_cast<const float4*>(src + 4);
        float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        bf16_t* dst;
        if (MODE == EPI_QKV) {
          if (n < p.n0) dst = p.out0 + (size_t)m * p.n0 + n;
          else if (n < p.n1) dst = p.out1 + (size_t)m * (p.n1 - p.n0) + (n - p.n0);
          else dst = p.out2 + (size_t)m * (p.N - p.n1) + (n - p.n1);
        } else if (MODE == EPI_SWIGLU) {
          dst = p.out0 + (size_t)m * p.ldo + n;
        } else {
          const uint4 h = hres[LOADS ? ph : 0][LOADS ? k : 0];
          const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            v[2 * e] += __uint_as_float(hw[e] << 16);
            v[2 * e + 1] += __uint_as_float(hw[e] & 0xffff0000u);
          }
          const int o = MODE == EPI_SCATTER ? orow[MODE == EPI_SCATTER ? ph : 0][MODE == EPI_SCATTER ? k : 0] : m;
          dst = p.out0 + (size_t)o * p.ldo + n;
        }
        *reinterpret_cast<uint4*>(dst) = make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]),
                                                    pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7]));
      }
      if (ph + 1 < NPH) lds_barrier();  // every thread has read the slabs the next phase overwrites
    }
  }
}

template <int MODE, bool DUAL, class TL, bool SK>
static kvb_status launch_bf16(hipStream_t st, const GemmArgs<bf16_t>& p, const SkArgs& sk, const char* name) {
  constexpr int OUT_N = DUAL ? TL::BN / 2 : TL::BN;
  const int tiles = cdiv(p.M_max, TL::BM) * cdiv(p.N, OUT_N);
  int per = (tiles * (SK ? sk.S : 1) + 7) / 8;
  if (SK && sk.xcd_blocks > 0) {
    per = 0;
    for (int x = 0; x < 8; x++) {
      int t0, nt, nh;
      mixed_run(tiles, x, sk.S, sk.xcd_blocks, t0, nt, nh);
      per = std::max(per, (nt - nh) * sk.S + nh * (sk.S + 1));
    }
  }
  dim3 grid(per * 8);
  {
    LaunchTimer lt(st, name, true);
    hipExtLaunchKernelGGL(gemm_bf16_kernel<MODE, DUAL, TL, SK>, grid, dim3(GEMM_THREADS), 0, st, lt.start(), lt.stop(),
                          0, p, sk);
  }
  return check_launch("gemm_bf16_kernel");
}

// Sum of a tile's split-K partials in slice order, then the epilogue of MODE;
// one thread per 8 consecutive output columns of a row.
template <int MODE, bool DUAL>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs<bf16_t> p, SkArgs sk) {
  const int M = row_count(p.n_rows, p.M_max);
  const int cpr = p.N / 8;
  const long c = (long)blockIdx.x * 256 + threadIdx.x;
  const int m = (int)(c / cpr), n = (int)(c % cpr) * 8;
  if (m >= M) return;
  int S = sk.S;
  if (sk.xcd_blocks > 0) {
    // this element's tile and the run of the mixed plan it sits in
    const int t = tile_index(m / sk.bm, n / sk.bn, sk.num_m, sk.num_n), tiles = sk.num_m * sk.num_n;
    for (int x = 0; x < 8; x++) {
      int t0, nt, nh;
      mixed_run(tiles, x, sk.S, sk.xcd_blocks, t0, nt, nh);
      if (t >= t0 && t < t0 + nt) S = sk.S + (t - t0 >= nt - nh ? 1 : 0);
    }
  }
  float v[8] = {}, u[8] = {};
  for (int s = 0; s < S; s++) {
    const float* src = sk.part + ((size_t)s * sk.rows + m) * sk.cols + n;
    const float4 a = *reinterpret_cast<const float4*>(src), b = *reinterpret_cast<const float4*>(src + 4);
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w; v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
    if (DUAL) {
      const float4 g = *reinterpret_cast<const float4*>(src + p.N), h = *reinterpret_cast<const float4*>(src + p.N + 4);
      u[0] += g.x; u[1] += g.y; u[2] += g.z; u[3] += g.w; u[4] += h.x; u[5] += h.y; u[6] += h.z; u[7] += h.w;
    }
  }
  bf16_t* dst;
  if (MODE == EPI_SWIGLU) {
#pragma unroll
    for (int e = 0; e < 8; e++) v[e] = DUAL ? silu_bf16(v[e]) * u[e] : v[e];
    dst = p.out0 + (size_t)m * p.ldo + n;
  } else if (MODE == EPI_QKV) {
    if (n < p.n0) dst = p.out0 + (size_t)m * p.n0 + n;
    else if (n < p.n1) dst = p.out1 + (size_t)m * (p.n1 - p.n0) + (n - p.n0);
    else dst = p.out2 + (size_t)m * (p.N - p.n1) + (n - p.n1);
  } else {
    const int rr = (MODE == EPI_RESID && p.resid_rows) ? p.resid_rows[m] : m;
    const uint4 h = *reinterpret_cast<const uint4*>(p.resid + (size_t)rr * p.ldr + n);
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
      v[2 * e] += __uint_as_float(hw[e] << 16);
      v[2 * e + 1] += __uint_as_float(hw[e] & 0xffff0000u);
    }
    const int orow = (MODE == EPI_SCATTER && p.out_rows) ? p.out_rows[m] : m;
    dst = p.out0 + (size_t)orow * p.ldo + n;
  }
  *reinterpret_cast<uint4*>(dst) =
      make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7]));
}

template <int MODE, bool DUAL>
static kvb_status launch_splitk_reduce(hipStream_t st, const GemmArgs<bf16_t>& p, const SkArgs& sk,
                                       const char* name) {
  const long n = (long)p.M_max * (p.N / 8);
  {
    LaunchTimer lt(st, name, true);
    hipExtLaunchKernelGGL(splitk_reduce_kernel<MODE, DUAL>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                          lt.start(), lt.stop(), 0, p, sk);
  }
  return check_launch("splitk_reduce_kernel");
}

// One-row product (M_max = 1, on launches that may split K, so no bitwise
// tie to the batched result is owed): the weights stream once from HBM and x
// sits in LDS.  Each wave owns GV_NW consecutive outputs (with SwiGLU their
// gate and up rows too); lane l takes the 16-byte chunks l, l + 64, ... of
// every row, four v_dot2_f32_bf16 per chunk, then one butterfly per row.  The
// epilogues are the tiled kernel's.
constexpr int GV_NW = 2, GV_WAVES = 4;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot8_bf16(const uint4& w, const uint4& x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), acc, false);
  return acc;
}

// RoPE epilogue of the one-row Q/K/V product (decode): the wave's two outputs
// are the pair (i, i + hd/2) of one head, rotated together; K and V also go to
// the row's slot in the pool.
struct RopeEpi {
  const int32_t* tok_pos;
  const int32_t* row_tok;
  const int32_t* dst_slot;
  bf16_t* k_pool;
  bf16_t* v_pool;
  int n_slots, Hkv, hd;
  RopeFreq rf;
};

// With NORM the row is RMS-normalised inside the product: while x is staged,
// each thread adds the squares of its elements and stores x * gain (rounded
// to bf16); the per-wave sums (in wave order) give 1 / rms, which scales the
// dot products in the epilogue.  This is the normalised product up to the
// rounding point of the scaled row, with no separate pass and no extra
// barrier.  p.a_rows, if set, picks the row of A.
// (at most 4 waves per SIMD: the registers for a whole batch of loads in flight)
template <int MODE, bool DUAL, bool ROPE = false, bool NORM = false>
__global__ void __launch_bounds__(64 * GV_WAVES) __attribute__((amdgpu_waves_per_eu(1, 4)))
gemv_bf16_kernel(GemmArgs<bf16_t> p, RopeEpi re) {
  static_assert(!ROPE || (MODE == EPI_QKV && !DUAL && GV_NW == 2), "RoPE pairs two Q/K/V outputs");
  static_assert(!NORM || MODE == EPI_QKV || MODE == EPI_SWIGLU, "the norm precedes Q/K/V and SwiGLU products");
  extern __shared__ __align__(16) uint8_t gv_x[];
  if (row_count(p.n_rows, p.M_max) < 1) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int C = p.K / 8;  // 16-byte chunks per row
  const int wg = blockIdx.x * GV_WAVES + wave;
  // the wave's outputs: nb + i (ROPE: the pair of one head, hd / 2 apart)
  const int nb = ROPE ? (wg / (re.hd / 2)) * re.hd + wg % (re.hd / 2) : wg * GV_NW;
  const int nstep = ROPE ? re.hd / 2 : 1;
  constexpr int R = DUAL ? 2 * GV_NW : GV_NW;  // rows i < GV_NW: B; the rest: B2
  constexpr int NB = 4;                        // 16-byte chunks per row in one batch of loads
  const uint4* wr[R];
#pragma unroll
  for (int i = 0; i < GV_NW; i++) {
    int n = nb + i * nstep < p.N ? nb + i * nstep : p.N - 1;
    n = n < 0 ? 0 : n;
    wr[i] = reinterpret_cast<const uint4*>(p.B + (size_t)n * p.K);
    if (DUAL) wr[GV_NW + i] = reinterpret_cast<const uint4*>(p.B2 + (size_t)n * p.K);
  }
  // batches of NB chunks per lane: all NB R weight loads of a batch issued
  // before any is used (eight chunks a batch ran 1 % slower over a decode
  // step); a lane adds its chunks in index order whatever the batching.
  // Streamed once: non-temporal, so the weights do not evict what the
  // neighbouring launches keep in L2.
  auto load_batch = [&](int c, uint4 (&w)[NB][R]) {
#pragma unroll
    for (int u = 0; u < NB; u++)
#pragma unroll
      for (int i = 0; i < R; i++) {
        const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(&wr[i][c + 64 * u]));
        w[u][i] = make_uint4(q.x, q.y, q.z, q.w);
      }
  };
  // the first batch is issued before x is staged: the weight stream does not
  // wait for the staging and its barrier
  const bool active = ROPE ? 2 * wg < p.N : nb < p.N;
  const bool first = active && lane + 64 * (NB - 1) < C;
  uint4 w0[NB][R];
  if (first) load_batch(lane, w0);

  const uint4* xg = reinterpret_cast<const uint4*>(p.A + (p.a_rows ? (size_t)p.a_rows[0] * p.K : 0));
  uint4* xs = reinterpret_cast<uint4*>(gv_x);
  float* red = reinterpret_cast<float*>(gv_x + (size_t)p.K * 2);  // NORM: the waves' sums of squares
  if constexpr (NORM) {
    // two chunks (and their gains) in flight per thread; squares in element order
    constexpr int TH = 64 * GV_WAVES;
    const uint4* gg = reinterpret_cast<const uint4*>(p.norm_w);
    float ss = 0.f;
    auto put = [&](int c, const uint4& v, const uint4& w) {
      float f[8], gf[8];
      unpack8(v, f);
      unpack8(w, gf);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        ss += f[e] * f[e];
        f[e] *= gf[e];
      }
      xs[c] = make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]),
                         pack2_bf16(f[6], f[7]));
    };
    const uint4 one = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);  // bf16 1.0 pairs
    for (int c = t; c < C; c += 2 * TH) {
      const bool two = c + TH < C;
      const uint4 v0 = xg[c], g0 = gg ? gg[c] : one;
      uint4 v1 = one, g1 = one;
      if (two) {
        v1 = xg[c + TH];
        g1 = gg ? gg[c + TH] : one;
      }
      put(c, v0, g0);
      if (two) put(c + TH, v1, g1);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
  } else {
    // four 16-byte loads in flight per thread, then the tail
    constexpr int TH = 64 * GV_WAVES;
    int c = t;
    for (; c + 3 * TH < C; c += 4 * TH) {
      const uint4 v0 = xg[c], v1 = xg[c + TH], v2 = xg[c + 2 * TH], v3 = xg[c + 3 * TH];
      xs[c] = v0;
      xs[c + TH] = v1;
      xs[c + 2 * TH] = v2;
      xs[c + 3 * TH] = v3;
    }
    for (; c < C; c += TH) xs[c] = xg[c];
  }
  __syncthreads();
  if (!active) return;
  float acc[R];
#pragma unroll
  for (int i = 0; i < R; i++) acc[i] = 0.f;
  auto use_batch = [&](int c, const uint4 (&w)[NB][R]) {
#pragma unroll
    for (int u = 0; u < NB; u++) {
      const uint4 xv = xs[c + 64 * u];
#pragma unroll
      for (int i = 0; i < R; i++) acc[i] = dot8_bf16(w[u][i], xv, acc[i]);
    }
  };
  int c = lane;
  if (first) {
    use_batch(c, w0);
    c += 64 * NB;
  }
  for (; c + 64 * (NB - 1) < C; c += 64 * NB) {
    uint4 w[NB][R];
    load_batch(c, w);
    __builtin_amdgcn_sched_group_barrier(0x020, NB * R, 0);  // every weight load of the batch first
    use_batch(c, w);
  }
  if (c < C) {
    // the last, partial batch: its chunks below C, all loads again before any use
    uint4 w[NB][R];
#pragma unroll
    for (int u = 0; u < NB; u++)
      if (c + 64 * u < C) {
#pragma unroll
        for (int i = 0; i < R; i++) {
          const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(&wr[i][c + 64 * u]));
          w[u][i] = make_uint4(q.x, q.y, q.z, q.w);
        }
      }
#pragma unroll
    for (int u = 0; u < NB; u++)
      if (c + 64 * u < C) {
        const uint4 xv = xs[c + 64 * u];
#pragma unroll
        for (int i = 0; i < R; i++) acc[i] = dot8_bf16(w[u][i], xv, acc[i]);
      }
  }
  float rs = 1.f;  // NORM: 1 / rms of the row
  if constexpr (NORM) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < GV_WAVES; w++) s += red[w];
    rs = 1.f / sqrtf(s / (float)p.K + p.eps);
  }
  if constexpr (ROPE) {
    // both sums in every lane; lane 0 stores the low half of the pair, lane 1
    // the high half.  Each value is first rounded to bf16, as the product
    // stores it, then rotated (Q, K) and rounded again, as the RoPE pass does.
    const float x0 = bf2f(f2bf(NORM ? wave_sum(acc[0]) * rs : wave_sum(acc[0])));
    const float x1 = bf2f(f2bf(NORM ? wave_sum(acc[1]) * rs : wave_sum(acc[1])));
    if (lane >= 2) return;
    const int n = nb + lane * nstep;
    float y = lane == 0 ? x0 : x1;
    if (nb < p.n1) {
      const int g = re.row_tok ? re.row_tok[0] : 0;
      const float2 cs = rope_cs(re.tok_pos[g], re.rf.f[nb % re.hd]);
      y = lane == 0 ? rot_lo(x0, x1, cs.x, cs.y) : rot_hi(x1, x0, cs.x, cs.y);
      y = bf2f(f2bf(y));
    }
    const bf16_t yb = f2bf(y);
    if (n < p.n0) {
      p.out0[n] = yb;
      return;
    }
    const bool is_k = n < p.n1;
    const int kn = is_k ? n - p.n0 : n - p.n1;
    (is_k ? p.out1 : p.out2)[kn] = yb;
    const int dst = re.dst_slot[0];
    if (dst >= 0 && dst < re.n_slots)
      (is_k ? re.k_pool : re.v_pool)[pool_off(dst, kn / re.hd, re.Hkv, re.hd) + kn % re.hd] = yb;
    return;
  }
  float v = 0.f, v2 = 0.f;
#pragma unroll
  for (int i = 0; i < GV_NW; i++) {
    float a = wave_sum(acc[i]);
    float b = DUAL ? wave_sum(acc[GV_NW + i]) : 0.f;
    if constexpr (NORM) {
      a *= rs;
      b *= rs;
    }
    if (lane == i) {
      v = a;
      v2 = b;
    }
  }
  const int n = nb + lane;
  if (lane >= GV_NW || n >= p.N) return;
  bf16_t* dst;
  if (MODE == EPI_SWIGLU) {
    v = DUAL ? silu_bf16(v) * v2 : v;
    dst = p.out0 + n;
  } else if (MODE == EPI_QKV) {
    if (n < p.n0) dst = p.out0 + n;
    else if (n < p.n1) dst = p.out1 + (n - p.n0);
    else dst = p.out2 + (n - p.n1);
  } else {
    const int rr = (MODE == EPI_RESID && p.resid_rows) ? p.resid_rows[0] : 0;
    v += bf2f(p.resid[(size_t)rr * p.ldr + n]);
    const int orow = (MODE == EPI_SCATTER && p.out_rows) ? p.out_rows[0] : 0;
    dst = p.out0 + (size_t)orow * p.ldo + n;
  }
  *dst = (bf16_t)(pack2_bf16(v, 0.f) & 0xffffu);
}

// the one-row product takes the row whole into LDS
static bool gemv_ok(const GemmArgs<bf16_t>& p) { return p.M_max == 1 && p.K % 8 == 0 && p.K <= 32768; }

template <int MODE, bool DUAL, bool ROPE = false, bool NORM = false>
static kvb_status launch_gemv(hipStream_t st, const GemmArgs<bf16_t>& p, const char* name, const RopeEpi& re = {}) {
  {
    LaunchTimer lt(st, name, true);
    hipExtLaunchKernelGGL(gemv_bf16_kernel<MODE, DUAL, ROPE, NORM>, dim3(cdiv(p.N, GV_NW * GV_WAVES)),
                          dim3(64 * GV_WAVES), (uint32_t)((size_t)p.K * 2 + (NORM ? 4 * GV_WAVES : 0)), st,
                          lt.start(), lt.stop(), 0, p, re);
  }
  return check_launch("gemv_bf16_kernel");
}

using TileL = Tile<256, 256, 2, 64, 2>;     // waves 128 x 64, 2 stages of K 64
using TileL192 = Tile<192, 256, 2, 64, 2>;  // waves 96 x 64
using TileM = Tile<256, 128, 4, 32, 4>;  // waves 64 x 64, 4 stages of K 32
using TileS = Tile<128, 128, 4, 32, 4>;  // waves 32 x 64, 4 stages of K 32
// few rows: 64-row tiles (waves 32 x 64, gate and up subtile pairs for
// SwiGLU) with a 4-stage ring, so each block keeps three 40 KiB stages of
// the weight stream in flight
using TileN = Tile<64, 256, 2, 64, 4>;

// split-K partials: float [S][rows][cols], at most this many bytes
constexpr size_t SK_BUDGET = (size_t)256 << 20;
size_t ws_gemm_sk_bytes(int) { return SK_BUDGET; }

// Launch choice.  Without split-K the per-element reduction order (K stages in
// order, 16-wide MFMA slices in order) is the same for every tile shape and
// stage depth, so picking the shape from the launch bound keeps every row's
// result independent of the batch.  `sk_ws` (SK_BUDGET bytes) allows split-K.
//
// Cost model (microseconds).  A block of BM x BN over K / S takes the longer
// of its MFMA work at 4.5 TFLOP/s x shape efficiency and its operand bytes at
// the rate one block streams them (150 GB/s for the large tiles, whose
// operands mostly hit L2; 60 GB/s for the 64-row tile, which streams the
// weights); whole waves of blocks run on the CUs; the launch takes at least
// its unique operand bytes at 5 TB/s; split-K adds the reduction launch, which
// reads the partials at 5 TB/s (their writes overlap the product's own work).
// A mixed split (some tiles S slices, some S + 1, whole rounds of blocks per
// XCD) is timed by placing each XCD's blocks in order on its CUs, each on the
// CU that frees first; the slowest XCD sets the time.

// time by which n_a blocks of length a, then n_b of length b, end on C CUs
static double greedy_finish(int C, int n_a, double a, int n_b, double b) {
  std::vector<double> cu(C, 0.0);
  double end = 0.0;
  for (int i = 0; i < n_a + n_b; i++) {
    std::pop_heap(cu.begin(), cu.end(), std::greater<double>());
    cu.back() += i < n_a ? a : b;
    end = std::max(end, cu.back());
    std::push_heap(cu.begin(), cu.end(), std::greater<double>());
  }
  return end;
}

template <int MODE, bool DUAL>
static kvb_status run_bf16(hipStream_t st, const GemmArgs<bf16_t>& p, const char* name, void* sk_ws = nullptr) {
  if (p.M_max == 0 || p.N == 0) return KVB_OK;
  // the loads address A and B with 32-bit byte offsets from their bases
  const size_t b_span = (DUAL ? (size_t)(p.B2 - p.B) + (size_t)p.N * p.K : (size_t)p.N * p.K) * 2;
  if (p.a_rows || (size_t)p.M_max * p.K * 2 > 0xffffffffu || b_span > 0xffffffffu)
    return fail(KVB_ERR_UNSUPPORTED, std::string(name) + ": operands beyond 4 GiB of one base");
  // one row on a launch that may split K: the weight-streaming product
  if (sk_ws && gemv_ok(p)) return launch_gemv<MODE, DUAL>(st, p, name);
  Ctx* c = current_ctx();
  const long cus = c ? c->n_cu : 256;
  struct Shape { int bm, bn, kb; double eff, rate; bool split; };
  const Shape shapes[5] = {{256, 256, 64, 1.0, 150e3, true},
                           {192, 256, 64, 0.95, 150e3, false},
                           {256, 128, 32, 0.85, 150e3, false},
                           {128, 128, 32, 0.65, 150e3, false},
                           {64, 256, 64, 0.5, 60e3, true}};
  const double cols = DUAL ? 2.0 * p.N : (double)p.N;
  const double hbm_us = (cols * p.K + (double)p.M_max * p.K) * 2.0 / 5e6;
  int best_shape = -1, best_s = 1, best_xb = 0;
  double best_t = 1e30;
  for (int si = 0; si < 5; si++) {
    const Shape& sh = shapes[si];
    if (p.K % sh.kb) continue;
    const long tiles = (long)cdiv(p.M_max, sh.bm) * cdiv(p.N, DUAL ? sh.bn / 2 : sh.bn);
    const int max_split = (sh.split && sk_ws && p.N % 8 == 0) ? 16 : 1;
    auto blk_us = [&](int S) {
      const double kk = (double)p.K / S;
      return std::max(2.0 * sh.bm * sh.bn * kk / (4.5e6 * sh.eff), (sh.bm + sh.bn) * kk * 2.0 / sh.rate);
    };
    for (int S = 1; S <= max_split && S <= p.K / sh.kb; S++) {
      if (S > 1 && (size_t)S * p.M_max * (size_t)cols * 4 > SK_BUDGET) break;
      double tt = std::max((double)((tiles * S + cus - 1) / cus) * blk_us(S), hbm_us);
      if (S > 1) tt += (double)S * p.M_max * cols * 4 / 5e6 + 4.0;
      if (tt < best_t * (S > 1 ? 0.92 : 1.0)) {
        best_t = tt;
        best_shape = si;
        best_s = S;
        best_xb = 0;
      }
      // mixed S / S + 1 filling the rounds the uniform S plan needs (up to 4)
      const long rounds = (tiles * S + cus - 1) / cus;
      if (S + 1 > max_split || S + 1 > p.K / sh.kb || cus % 8 || rounds > 4 || tiles < 8 ||
          (size_t)(S + 1) * p.M_max * (size_t)cols * 4 > SK_BUDGET)
        continue;
      const int C = (int)(cus / 8), xb = (int)(rounds * C);
      double mk = 0.0;
      long extra = 0;
      for (int x = 0; x < 8; x++) {
        int t0, nt, nh;
        mixed_run((int)tiles, x, S, xb, t0, nt, nh);
        mk = std::max(mk, greedy_finish(C, (nt - nh) * S, blk_us(S), nh * (S + 1), blk_us(S + 1)));
        extra += nh;
      }
      if (extra == 0) continue;
      tt = std::max(mk, hbm_us) + (S + (double)extra / tiles) * p.M_max * cols * 4 / 5e6 + 4.0;
      if (tt < best_t * 0.92) {
        best_t = tt;
        best_shape = si;
        best_s = S;
        best_xb = xb;
      }
    }
  }
  SkArgs sk{};
  sk.S = 1;
  if (best_s > 1 || best_xb > 0) {
    sk.S = best_s;
    sk.rows = p.M_max;  // partial row stride; only rows below the row count are written
    sk.cols = DUAL ? 2 * p.N : p.N;
    sk.part = (float*)sk_ws;
    sk.xcd_blocks = best_xb;
    sk.bm = shapes[best_shape].bm;
    sk.bn = DUAL ? shapes[best_shape].bn / 2 : shapes[best_shape].bn;
    sk.num_m = cdiv(p.M_max, sk.bm);
    sk.num_n = cdiv(p.N, sk.bn);
    if (best_shape == 0) KVB_TRY((launch_bf16<MODE, DUAL, TileL, true>(st, p, sk, name)));
    else KVB_TRY((launch_bf16<MODE, DUAL, TileN, true>(st, p, sk, name)));
    return launch_splitk_reduce<MODE, DUAL>(st, p, sk, "splitk_reduce");
  }
  switch (best_shape) {
    case 0: return launch_bf16<MODE, DUAL, TileL, false>(st, p, sk, name);
    case 1: return launch_bf16<MODE, DUAL, TileL192, false>(st, p, sk, name);
    case 2: return launch_bf16<MODE, DUAL, TileM, false>(st, p, sk, name);
    case 3: return launch_bf16<MODE, DUAL, TileS, false>(st, p, sk, name);
    case 4: return launch_bf16<MODE, DUAL, TileN, false>(st, p, sk, name);
    default: return fail(KVB_ERR_UNSUPPORTED, std::string(name) + ": K must be a multiple of 32");
  }
}

// ====================================================================== fp32 FMA

constexpr int FB = 64, FK = 16;

template <int MODE, bool DUAL, bool NORM>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs<float> p) {
  __shared__ float sA[FK][FB + 4];
  __shared__ float sB[FK][FB + 4];
  __shared__ float sB2[DUAL ? FK : 1][FB + 4];
  __shared__ float s_rinv[FB];
  __shared__ int s_arow[FB];
  const int M = row_count(p.n_rows, p.M_max);
  const int m0 = blockIdx.x * FB, n0 = blockIdx.y * FB;
  if (m0 >= M) return;
  const int t = threadIdx.x;
  if (t < FB) {
    int m = m0 + t;
    m = m < M ? m : M - 1;
    s_arow[t] = p.a_rows ? p.a_rows[m] : m;
  }
  __syncthreads();
  if (NORM) {
    // 4 threads per row, each a strided partial sum, combined in fixed order
    const int r = t >> 2, q = t & 3;
    const float* a = p.A + (size_t)s_arow[r] * p.K;
    float s = 0.f;
    for (int k = q; k < p.K; k += 4) s += a[k] * a[k];
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (q == 0) s_rinv[r] = 1.f / sqrtf(s / (float)p.K + p.eps);
    __syncthreads();
  }
  const int tr = (t >> 4) * 4, tc = (t & 15) * 4;
  float acc[4][4] = {}, acc2[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += FK) {
    for (int i = t; i < FB * FK; i += 256) {
      const int r = i / FK, kk = i % FK, k = k0 + kk;
      float a = 0.f, b = 0.f, b2 = 0.f;
      if (k < p.K) {
        a = p.A[(size_t)s_arow[r] * p.K + k];
        if (NORM && p.norm_w) a *= p.norm_w[k];
        int n = n0 + r;
        n = n < p.N ? n : p.N - 1;
        b = p.B[(size_t)n * p.K + k];
        if (DUAL) b2 = p.B2[(size_t)n * p.K + k];
      }
      sA[kk][r] = a;
      sB[kk][r] = b;
      if (DUAL) sB2[kk][r] = b2;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; kk++) {
      float av[4], bv[4], bv2[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        av[i] = sA[kk][tr + i];
        bv[i] = sB[kk][tc + i];
        if (DUAL) bv2[i] = sB2[kk][tc + i];
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
          if (DUAL) acc2[i][j] = fmaf(av[i], bv2[j], acc2[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int m = m0 + tr + i;
    if (m >= M) continue;
    const float rinv = NORM ? s_rinv[tr + i] : 1.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int n = n0 + tc + j;
      if (n < p.N) epilogue<MODE, float>(p, m, n, acc[i][j], DUAL ? acc2[i][j] : 0.f, rinv);
    }
  }
}

template <int MODE, bool DUAL, bool NORM>
static kvb_status run_f32(hipStream_t st, const GemmArgs<float>& p, const char* name) {
  if (p.M_max == 0 || p.N == 0) return KVB_OK;
  dim3 grid(cdiv(p.M_max, FB), cdiv(p.N, FB));
  {
    LaunchTimer lt(st, name);
    gemm_f32_kernel<MODE, DUAL, NORM><<<grid, 256, 0, st>>>(p);
  }
  return check_launch("gemm_f32_kernel");
}

template <class T>
kvb_status launch_rope(hipStream_t st, int T_max, const int32_t* n_rows, const int32_t* row_tok,
                       const int32_t* tok_pos, void* q, void* k, const kvb_model_desc* d);

template <class T>
static kvb_status qkv_impl(hipStream_t st, const kvb_model_desc* d, int T_max, const int32_t* n_rows,
                           const int32_t* row_tok, const void* hidden, const void* norm_w, const void* w_qkv,
                           const int32_t* tok_pos, void* q, void* k, void* v, void* ws, bool split_k) {
  GemmArgs<T> p{};
  p.B = (const T*)w_qkv;
  p.M_max = T_max;
  p.n_rows = n_rows;
  p.K = d->d_model;
  p.n0 = d->n_q_heads * d->head_dim;
  p.n1 = p.n0 + d->n_kv_heads * d->head_dim;
  p.N = p.n1 + d->n_kv_heads * d->head_dim;
  p.eps = d->rms_eps;
  p.out0 = (T*)q;
  p.out1 = (T*)k;
  p.out2 = (T*)v;
  if constexpr (sizeof(T) == 2) {
    if (split_k && T_max == 1 && gemv_ok(p)) {
      // one row: the norm inside the weight-streaming product
      p.A = (const T*)hidden;
      p.a_rows = row_tok;
      p.norm_w = (const T*)norm_w;
      KVB_TRY((launch_gemv<EPI_QKV, false, false, true>(st, p, "gemm_qkv")));
      if (tok_pos) return launch_rope<T>(st, T_max, n_rows, row_tok, tok_pos, q, k, d);
      return KVB_OK;
    }
    // normalised rows a [T, d] in workspace, then a plain GEMM
    bf16_t* a = (bf16_t*)ws;
    KVB_TRY(rmsnorm_rows(st, (const bf16_t*)hidden, row_tok, n_rows, T_max, d->d_model, (const bf16_t*)norm_w,
                         d->rms_eps, a));
    p.A = a;
    // split-K partials after the normalised rows, only when the caller allows it
    void* sk_ws = split_k ? (void*)((char*)ws + ws_qkv_bytes(d, T_max)) : nullptr;
    KVB_TRY((run_bf16<EPI_QKV, false>(st, p, "gemm_qkv", sk_ws)));
  } else {
    p.A = (const T*)hidden;
    p.a_rows = row_tok;
    p.norm_w = (const T*)norm_w;
    KVB_TRY((run_f32<EPI_QKV, false, true>(st, p, "gemm_qkv")));
  }
  if (tok_pos) return launch_rope<T>(st, T_max, n_rows, row_tok, tok_pos, q, k, d);
  return KVB_OK;
}

kvb_status qkv_rope_one_row(hipStream_t st, const kvb_model_desc* d, const int32_t* n_rows, const int32_t* row_tok,
                            const void* hidden, const void* norm_w, const void* w_qkv, const int32_t* tok_pos, void* q,
                            void* k, void* v, void* k_pool, void* v_pool, int n_slots, const int32_t* dst_slot,
                            void* ws) {
  GemmArgs<bf16_t> p{};
  p.B = (const bf16_t*)w_qkv;
  p.M_max = 1;
  p.n_rows = n_rows;
  p.K = d->d_model;
  p.n0 = d->n_q_heads * d->head_dim;
  p.n1 = p.n0 + d->n_kv_heads * d->head_dim;
  p.N = p.n1 + d->n_kv_heads * d->head_dim;
  p.eps = d->rms_eps;
  p.out0 = (bf16_t*)q;
  p.out1 = (bf16_t*)k;
  p.out2 = (bf16_t*)v;
  (void)ws;
  p.A = (const bf16_t*)hidden;  // normalised inside the product
  p.a_rows = row_tok;
  p.norm_w = (const bf16_t*)norm_w;
  RopeEpi re{};
  re.tok_pos = tok_pos;
  re.row_tok = row_tok;
  re.dst_slot = dst_slot;
  re.k_pool = (bf16_t*)k_pool;
  re.v_pool = (bf16_t*)v_pool;
  re.n_slots = n_slots;
  re.Hkv = d->n_kv_heads;
  re.hd = d->head_dim;
  re.rf = rope_freq(d->head_dim, d->rope_base);
  return launch_gemv<EPI_QKV, false, true, true>(st, p, "gemm_qkv", re);
}

template <class T>
static kvb_status mlp_impl(hipStream_t st, const kvb_model_desc* d, int T_max, const int32_t* n_rows,
                           const int32_t* row_tok, const void* attn_o, const void* w_o, void* hidden,
                           const void* norm2_w, const void* w_gate_up, const void* w_down, void* ws) {
  const int D = d->d_model, F = d->ffn, QD = d->n_q_heads * d->head_dim;
  // workspace: h1 [T, d], u [T, F], then (bf16) the normalised h1 [T, d]
  const size_t h1_bytes = align_up((size_t)T_max * D * sizeof(T), 256);
  T* h1 = (T*)ws;
  T* u = (T*)((char*)ws + h1_bytes);
  T* hn = (T*)((char*)ws + h1_bytes + align_up((size_t)T_max * F * sizeof(T), 256));
  void* sk_ws = (char*)hn + ws_qkv_bytes(d, T_max);  // stream-K partials (bf16)
  // h1 = hidden[row] + o W_o^T
  GemmArgs<T> a{};
  a.A = (const T*)attn_o;
  a.B = (const T*)w_o;
  a.M_max = T_max;
  a.n_rows = n_rows;
  a.N = D;
  a.K = QD;
  a.out0 = h1;
  a.ldo = D;
  a.resid = (const T*)hidden;
  a.resid_rows = row_tok;
  a.ldr = D;
  // u = silu(RMSNorm(h1) W_gate^T) * (RMSNorm(h1) W_up^T)
  GemmArgs<T> b{};
  b.A = h1;
  b.B = (const T*)w_gate_up;
  b.B2 = (const T*)w_gate_up + (size_t)F * D;
  b.norm_w = (const T*)norm2_w;
  b.M_max = T_max;
  b.n_rows = n_rows;
  b.N = F;
  b.K = D;
  b.eps = d->rms_eps;
  b.out0 = u;
  b.ldo = F;
  // hidden[row] = h1 + u W_down^T
  GemmArgs<T> c{};
  c.A = u;
  c.B = (const T*)w_down;
  c.M_max = T_max;
  c.n_rows = n_rows;
  c.N = D;
  c.K = F;
  c.out0 = (T*)hidden;
  c.ldo = D;
  c.resid = h1;
  c.ldr = D;
  c.out_rows = row_tok;
  if constexpr (sizeof(T) == 2) {
    KVB_TRY((run_bf16<EPI_RESID, false>(st, a, "gemm_oproj", sk_ws)));
    if (gemv_ok(b)) {
      // one row: the norm inside the weight-streaming product
      KVB_TRY((launch_gemv<EPI_SWIGLU, true, false, true>(st, b, "gemm_swiglu")));
      return run_bf16<EPI_SCATTER, false>(st, c, "gemm_down", sk_ws);
    }
    KVB_TRY(rmsnorm_rows(st, h1, nullptr, n_rows, T_max, D, (const bf16_t*)norm2_w, d->rms_eps, hn));
    b.A = hn;
    b.norm_w = nullptr;
    KVB_TRY((run_bf16<EPI_SWIGLU, true>(st, b, "gemm_swiglu", sk_ws)));
    return run_bf16<EPI_SCATTER, false>(st, c, "gemm_down", sk_ws);
  } else {
    KVB_TRY((run_f32<EPI_RESID, false, false>(st, a, "gemm_oproj")));
    KVB_TRY((run_f32<EPI_SWIGLU, true, true>(st, b, "gemm_swiglu")));
    return run_f32<EPI_SCATTER, false, false>(st, c, "gemm_down");
  }
}

}  // namespace kvb

using namespace kvb;

extern "C" kvb_status kvb_qkv_proj(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                                   const int32_t* n_rows, const int32_t* row_tok, const void* hidden,
                                   const void* norm_w, const void* w_qkv, const int32_t* tok_pos, void* q, void* k,
                                   void* v, void* ws, size_t ws_bytes, int32_t flags) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0) return fail(KVB_ERR_INVALID_ARG, "T_max < 0");
  if (flags != KVB_QKV_BATCH_INVARIANT && flags != KVB_QKV_SPLIT_K) return fail(KVB_ERR_INVALID_ARG, "bad flags");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(hidden, "hidden");
  KVB_CHECK_PTR(w_qkv, "w_qkv");
  KVB_CHECK_PTR(q, "q");
  KVB_CHECK_PTR(k, "k");
  KVB_CHECK_PTR(v, "v");
  const bool split_k = flags == KVB_QKV_SPLIT_K && desc->dtype == KVB_BF16;
  const size_t need = ws_qkv_bytes(desc, T_max) + (split_k ? ws_gemm_sk_bytes(0) : 0);
  if (need && (!ws || ws_bytes < need)) return fail(KVB_ERR_WORKSPACE, "kvb_qkv_proj workspace too small");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  if (desc->dtype == KVB_BF16)
    return qkv_impl<bf16_t>(st, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v, ws, split_k);
  return qkv_impl<float>(st, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v, ws, false);
}

extern "C" kvb_status kvb_mlp(kvb_ctx* ctx, void* stream, const kvb_model_desc* desc, int32_t T_max,
                              const int32_t* n_rows, const int32_t* row_tok, const void* attn_o, const void* w_o,
                              void* hidden, const void* norm2_w, const void* w_gate_up, const void* w_down, void* ws,
                              size_t ws_bytes) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0) return fail(KVB_ERR_INVALID_ARG, "T_max < 0");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(attn_o, "attn_o");
  KVB_CHECK_PTR(w_o, "w_o");
  KVB_CHECK_PTR(hidden, "hidden");
  KVB_CHECK_PTR(w_gate_up, "w_gate_up");
  KVB_CHECK_PTR(w_down, "w_down");
  if (!ws || ws_bytes < ws_mlp_bytes(desc, T_max, reinterpret_cast<Ctx*>(ctx)->n_cu))
    return fail(KVB_ERR_WORKSPACE, "kvb_mlp workspace too small");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  if (desc->dtype == KVB_BF16)
    return mlp_impl<bf16_t>(st, desc, T_max, n_rows, row_tok, attn_o, w_o, hidden, norm2_w, w_gate_up, w_down, ws);
  return mlp_impl<float>(st, desc, T_max, n_rows, row_tok, attn_o, w_o, hidden, norm2_w, w_gate_up, w_down, ws);
}
