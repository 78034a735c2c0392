// Gathered-row GEMMs of the link step: the Q/K/V projection and the output
// projection + SwiGLU MLP of the recomputed rows (EPIC page, section 4,
// LegoLink steps 2 and 5; the same per-layer dataflow serves CacheSlide).
//
//   C[m, n] = sum_k A[row(m), k] * W[n, k]      (W is [N, K], row-major)
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 on gfx950, 128x128x64 block tiles,
// 4 waves of 64x64, LDS double buffering with a register prefetch of the next
// K tile.  fp32 path: an LDS-tiled FMA kernel with the same prologue and
// epilogues (used by the small float32 workload).
//
// Fusions: RMSNorm of the A rows is folded in (sum of squares accumulated
// while the tiles stream through, 1/rms applied in the epilogue, gains applied
// to A before it reaches the matrix cores); epilogues split Q/K/V, add the
// residual, apply SiLU(gate) * up on a dual-B tile, or scatter rows back to
// the hidden buffer.
//
// Row invariance: the reduction order of every output element (K tiles in
// order, the MFMA's k slices in order) and of every row's sum of squares (a
// fixed thread-to-k-chunk assignment reduced by xor shuffles) depends only on
// k, never on the row's index or on M, so a row's result is the same whatever
// batch it is computed in.
#include "common.h"

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
// Block = 4 waves in a 2 x 2 grid; wave tile = (32 TM) x (32 TN) outputs as
// TM x TN tiles of v_mfma_f32_32x32x16_bf16; block tile BM = 64 TM rows of A
// and BN = 64 TN rows of B.  K advances 32 at a time through a ring of four
// LDS stages filled by direct-to-LDS loads (global_load_lds_dwordx4) three
// stages ahead, so global latency is hidden without staging registers.
//
// LDS stage layout: rows of 64 bytes (32 bf16 = four 16-byte chunks); chunk c
// of row r is stored at position c ^ ((r >> 2) & 3), which makes the 16-byte
// fragment reads of 16 consecutive rows hit 16 distinct bank groups.  A wave's
// load instruction fills 1 KiB = 16 rows; its lane j fetches row j / 4, chunk
// (j % 4) ^ swizzle(row), and lands at position j % 4.
//
// SwiGLU (DUAL): the B tile interleaves 32-row subtiles of the gate and up
// matrices (gate cols c..c+31, up cols c..c+31, ...), so a wave holds gate
// and up of the same outputs in neighbouring accumulators; BN/2 outputs wide.
//
// RMSNorm is not fused here: rmsnorm_rows_kernel writes the normalised rows
// (bf16, one rounding) to workspace and the GEMM reads them as a plain A.
// Carrying the row sums and the gains through the K loop cost registers that
// the 4 x 4 tile does not have.

constexpr int KB = 32;          // K per stage
constexpr int NSTAGE = 4;       // LDS ring depth (prefetch distance 3)
constexpr int GEMM_THREADS = 256;

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

static kvb_status rmsnorm_rows(hipStream_t st, const bf16_t* x, const int32_t* a_rows, const int32_t* n_rows,
                               int T_max, int K, const bf16_t* g, float eps, bf16_t* y) {
  {
    LaunchTimer lt(st, "rmsnorm");
    rmsnorm_rows_kernel<<<cdiv(T_max, 4), 256, 0, st>>>(x, a_rows, n_rows, T_max, K, g, eps, y);
  }
  return check_launch("rmsnorm_rows_kernel");
}

template <int TM, int TN>
struct Tile {
  static constexpr int BM = 64 * TM, BN = 64 * TN;
  static constexpr int A_I = BM / 64, B_I = BN / 64;  // load instructions per wave per stage
  static constexpr int PER = A_I + B_I;
  static constexpr int STAGE_BYTES = (BM + BN) * 64;
  static constexpr int EPI_BYTES = 32 * (BN + 8) * 4;  // one 32-row epilogue phase
  static constexpr int ARR = STAGE_BYTES > EPI_BYTES ? STAGE_BYTES : EPI_BYTES;
};

// The four ring stages are separate LDS objects and the K loop is unrolled by
// four, so the compiler can see that a stage being read is not the one the
// in-flight loads are filling (one shared object would make it drain every
// outstanding load before each LDS read).
template <int TM, int TN, int S>
struct StageLds {
  __device__ static uint8_t* ptr() {
    __shared__ __align__(16) uint8_t buf[Tile<TM, TN>::ARR];
    return buf;
  }
};

template <int MODE, bool DUAL, int TM, int TN>
__global__ void __launch_bounds__(GEMM_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bf16_kernel(GemmArgs<bf16_t> p) {
  using TL = Tile<TM, TN>;
  constexpr int BM = TL::BM, BN = TL::BN, A_I = TL::A_I, B_I = TL::B_I, PER = TL::PER;
  constexpr int OUT_N = DUAL ? BN / 2 : BN;  // output columns per block
  uint8_t* const stg[NSTAGE] = {StageLds<TM, TN, 0>::ptr(), StageLds<TM, TN, 1>::ptr(), StageLds<TM, TN, 2>::ptr(),
                                StageLds<TM, TN, 3>::ptr()};

  const int M = row_count(p.n_rows, p.M_max);
  // Tile rasterisation.  Workgroups go to the 8 XCDs round-robin (id % 8), each
  // XCD with its own L2: give every XCD a contiguous run of a grouped tile
  // order (GM m-tiles sweeping all n-tiles), so the tiles an XCD runs at the
  // same time share A and B panels in its L2.
  int tm, tn;
  {
    const int num_m = cdiv_dev(p.M_max, BM), num_n = cdiv_dev(p.N, OUT_N);
    const int total = num_m * num_n;
    const int per = (total + 7) >> 3;
    const int tid = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (tid >= total) return;
    const int GM = num_m <= 16 ? num_m : 8;
    const int gsize = GM * num_n;
    const int grp = tid / gsize, first = grp * GM;
    const int gm = min(GM, num_m - first);
    const int in = tid - grp * gsize;
    tm = first + in % gm;
    tn = in / gm;
  }
  const int m0 = tm * BM, n0 = tn * OUT_N;
  if (m0 >= M) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = (wave >> 1) * (32 * TM), wn = (wave & 1) * (32 * TN);

  // ---- direct-to-LDS loaders: instruction i of this wave covers tile rows
  //      (wave * X_I + i) * 16 + lane / 4, lane position lane % 4
  const int lrow = lane >> 2, lpos = lane & 3;
  const bf16_t* a_src[A_I];
  const bf16_t* b_src[B_I];
#pragma unroll
  for (int i = 0; i < A_I; i++) {
    const int r = (wave * A_I + i) * 16 + lrow;
    int m = m0 + r;
    m = m < M ? m : M - 1;
    const int ar = p.a_rows ? p.a_rows[m] : m;
    a_src[i] = p.A + (size_t)ar * p.K + ((lpos ^ ((r >> 2) & 3)) * 8);
  }
#pragma unroll
  for (int i = 0; i < B_I; i++) {
    const int r = (wave * B_I + i) * 16 + lrow;  // B-tile row; 32-row subtile r / 32
    const bf16_t* base = p.B;
    int n;
    if (DUAL) {
      base = ((r >> 5) & 1) ? p.B2 : p.B;
      n = n0 + (r >> 6) * 32 + (r & 31);
    } else {
      n = n0 + r;
    }
    n = n < p.N ? n : p.N - 1;
    b_src[i] = base + (size_t)n * p.K + ((lpos ^ ((r >> 2) & 3)) * 8);
  }
  const int KT = p.K / KB;
#define KVB_ISSUE(KT_, ST_)                                                                       \
  do {                                                                                            \
    uint8_t* st_ = (ST_);                                                                         \
    const int ko_ = (KT_) * KB;                                                                   \
    _Pragma("unroll") for (int i = 0; i < A_I; i++)                                               \
      dma16(a_src[i] + ko_, __builtin_amdgcn_readfirstlane(lds_addr(st_ + (wave * A_I + i) * 1024))); \
    _Pragma("unroll") for (int i = 0; i < B_I; i++)                                               \
      dma16(b_src[i] + ko_, __builtin_amdgcn_readfirstlane(lds_addr(st_ + BM * 64 + (wave * B_I + i) * 1024))); \
  } while (0)

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = (f32x16_t){};

  // fragment addressing: lane reads row (l % 32) of a 32-row subtile, chunk 2 s + l / 32
  const int fr = lane & 31, fh = lane >> 5, fswz = (fr >> 2) & 3;
  const int foff0 = fr * 64 + (((0 + fh) ^ fswz) * 16);  // k16 step 0
  const int foff1 = fr * 64 + (((2 + fh) ^ fswz) * 16);  // k16 step 1

  // Fragments are double-buffered in registers: while the MFMAs of one k16
  // step run, the reads of the next step (in the same stage, or step 0 of the
  // next stage) are in flight.  Stage kt+1 is therefore published (vmcnt wait
  // + barrier) at the start of step kt, and the ring is refilled three stages
  // ahead into the stage consumed in the previous step.
  uint4 fa[2][TM], fb[2][TN];
#define KVB_FRAGS(BUF, STG, FO)                                                                   \
  do {                                                                                            \
    const uint8_t* sa_ = (STG) + wm * 64 + (FO);                                                  \
    const uint8_t* sb_ = (STG) + BM * 64 + wn * 64 + (FO);                                        \
    _Pragma("unroll") for (int i = 0; i < TM; i++) fa[BUF][i] = *reinterpret_cast<const uint4*>(sa_ + i * 2048); \
    _Pragma("unroll") for (int j = 0; j < TN; j++) fb[BUF][j] = *reinterpret_cast<const uint4*>(sb_ + j * 2048); \
  } while (0)
#define KVB_MMA(BUF)                                                                              \
  do {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < TM; i++)                                                \
      _Pragma("unroll") for (int j = 0; j < TN; j++)                                              \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[BUF][i]), as_bf16x8(fb[BUF][j]), acc[i][j], 0, 0, 0); \
  } while (0)
  // one K step on ring stage S (compile-time), with stage S+1 published on entry
#define KVB_STEP(S, KT_)                                                                          \
  do {                                                                                            \
    const int kt_ = (KT_);                                                                        \
    if (kt_ + 2 < KT) wait_vmcnt<PER>();                                                          \
    else wait_vmcnt<0>();                                                                         \
    lds_barrier();                                                                                \
    if (kt_ + 3 < KT) KVB_ISSUE(kt_ + 3, stg[((S) + 3) & 3]);                                     \
    KVB_FRAGS(1, stg[S], foff1);                                                                  \
    KVB_MMA(0);                                                                                   \
    if (kt_ + 1 < KT) KVB_FRAGS(0, stg[((S) + 1) & 3], foff0);                                    \
    KVB_MMA(1);                                                                                   \
  } while (0)

  if (KT > 0) KVB_ISSUE(0, stg[0]);
  if (KT > 1) KVB_ISSUE(1, stg[1]);
  if (KT > 2) KVB_ISSUE(2, stg[2]);
  // publish stage 0, read its step-0 fragments
  if (KT > 2) wait_vmcnt<2 * PER>();
  else if (KT > 1) wait_vmcnt<PER>();
  else wait_vmcnt<0>();
  lds_barrier();
  if (KT > 0) KVB_FRAGS(0, stg[0], foff0);
  int kt = 0;
  for (; kt + 4 <= KT; kt += 4) {
    KVB_STEP(0, kt);
    KVB_STEP(1, kt + 1);
    KVB_STEP(2, kt + 2);
    KVB_STEP(3, kt + 3);
  }
  if (kt < KT) KVB_STEP(0, kt);
  if (kt + 1 < KT) KVB_STEP(1, kt + 1);
  if (kt + 2 < KT) KVB_STEP(2, kt + 2);
#undef KVB_STEP
#undef KVB_MMA
#undef KVB_FRAGS
#undef KVB_ISSUE
  wait_vmcnt<0>();
  lds_barrier();  // every wave is done with the ring before the epilogue reuses LDS

  // Epilogue, staged through LDS in 2 TM phases of 32 rows: the two waves
  // owning a phase's rows (subtile i of their half) write their float
  // accumulators (SwiGLU already combined) to a [32][OUT_N] tile, then all
  // threads read 8 consecutive outputs of a row, apply the mode (scale,
  // residual, scatter) and store 16 bytes at a time.
  // acc[i][j][r] sits at tile row wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,
  // tile col wn + 32 j + lane % 32 (DUAL: output col (wn / 32 + j) / 2 * 32 + lane % 32).
  constexpr int LDC = OUT_N + 8;  // floats; rows 4 apart land 32 banks apart
  float* sC = reinterpret_cast<float*>(stg[0]);
  const int lc = lane & 31;
#pragma unroll
  for (int ph = 0; ph < 2 * TM; ph++) {
    const int i = ph % TM;
    if ((wave >> 1) == ph / TM) {
#pragma unroll
      for (int j = 0; j < TN; j += (DUAL ? 2 : 1)) {
        const int cl = DUAL ? ((wn / 32 + j) >> 1) * 32 + lc : wn + j * 32 + lc;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int rl = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);  // row inside the phase
          float v = acc[i][j][r];
          if (DUAL) v = silu(v) * acc[i][j + 1][r];
          sC[rl * LDC + cl] = v;
        }
      }
    }
    __syncthreads();
    constexpr int CPR = OUT_N / 8;  // 8-output chunks per row
    for (int c = t; c < 32 * CPR; c += GEMM_THREADS) {
      const int rl = c / CPR, cc = (c % CPR) * 8;
      const int ml = ph * 32 + rl, m = m0 + ml, n = n0 + cc;
      if (m >= M || n >= p.N) continue;
      const float4 lo = *reinterpret_cast<const float4*>(sC + rl * LDC + cc);
      const float4 hi = *reinterpret_cast<const float4*>(sC + rl * LDC + cc + 4);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      bf16_t* dst;
      if (MODE == EPI_QKV) {
        if (n < p.n0) dst = p.out0 + (size_t)m * p.n0 + n;
        else if (n < p.n1) dst = p.out1 + (size_t)m * (p.n1 - p.n0) + (n - p.n0);
        else dst = p.out2 + (size_t)m * (p.N - p.n1) + (n - p.n1);
      } else if (MODE == EPI_SWIGLU) {
        dst = p.out0 + (size_t)m * p.ldo + n;
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
      *reinterpret_cast<uint4*>(dst) = make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]),
                                                  pack2_bf16(v[6], v[7]));
    }
    __syncthreads();
  }
}

template <int MODE, bool DUAL, int TM, int TN>
static kvb_status launch_bf16(hipStream_t st, const GemmArgs<bf16_t>& p, const char* name) {
  using TL = Tile<TM, TN>;
  constexpr int OUT_N = DUAL ? TL::BN / 2 : TL::BN;
  const int total = cdiv(p.M_max, TL::BM) * cdiv(p.N, OUT_N);
  dim3 grid(((total + 7) / 8) * 8);
  {
    LaunchTimer lt(st, name);
    gemm_bf16_kernel<MODE, DUAL, TM, TN><<<grid, GEMM_THREADS, 0, st>>>(p);
  }
  return check_launch("gemm_bf16_kernel");
}

// Tile choice: the per-element reduction order (32-wide K stages, 16-wide MFMA
// slices in order) is the same for every tile shape, so picking the shape from
// the launch bound keeps every row's result independent of the batch.
template <int MODE, bool DUAL>
static kvb_status run_bf16(hipStream_t st, const GemmArgs<bf16_t>& p, const char* name) {
  if (p.M_max == 0 || p.N == 0) return KVB_OK;
  const Ctx* c = current_ctx();
  const long cus = c ? c->n_cu : 256;
  const long big_blocks = (long)cdiv(p.M_max, 256) * cdiv(p.N, DUAL ? 128 : 256);
  if (big_blocks >= cus) return launch_bf16<MODE, DUAL, 4, 4>(st, p, name);
  const long mid_blocks = (long)cdiv(p.M_max, 256) * cdiv(p.N, DUAL ? 64 : 128);
  if (mid_blocks >= cus) return launch_bf16<MODE, DUAL, 4, 2>(st, p, name);
  return launch_bf16<MODE, DUAL, 2, 2>(st, p, name);
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
                           const int32_t* tok_pos, void* q, void* k, void* v, void* ws) {
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
    // normalised rows a [T, d] in workspace, then a plain GEMM
    bf16_t* a = (bf16_t*)ws;
    KVB_TRY(rmsnorm_rows(st, (const bf16_t*)hidden, row_tok, n_rows, T_max, d->d_model, (const bf16_t*)norm_w,
                         d->rms_eps, a));
    p.A = a;
    KVB_TRY((run_bf16<EPI_QKV, false>(st, p, "gemm_qkv")));
  } else {
    p.A = (const T*)hidden;
    p.a_rows = row_tok;
    p.norm_w = (const T*)norm_w;
    KVB_TRY((run_f32<EPI_QKV, false, true>(st, p, "gemm_qkv")));
  }
  if (tok_pos) return launch_rope<T>(st, T_max, n_rows, row_tok, tok_pos, q, k, d);
  return KVB_OK;
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
    KVB_TRY((run_bf16<EPI_RESID, false>(st, a, "gemm_oproj")));
    KVB_TRY(rmsnorm_rows(st, h1, nullptr, n_rows, T_max, D, (const bf16_t*)norm2_w, d->rms_eps, hn));
    b.A = hn;
    b.norm_w = nullptr;
    KVB_TRY((run_bf16<EPI_SWIGLU, true>(st, b, "gemm_swiglu")));
    return run_bf16<EPI_SCATTER, false>(st, c, "gemm_down");
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
                                   void* v, void* ws, size_t ws_bytes) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0) return fail(KVB_ERR_INVALID_ARG, "T_max < 0");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(hidden, "hidden");
  KVB_CHECK_PTR(w_qkv, "w_qkv");
  KVB_CHECK_PTR(q, "q");
  KVB_CHECK_PTR(k, "k");
  KVB_CHECK_PTR(v, "v");
  const size_t need = ws_qkv_bytes(desc, T_max);
  if (need && (!ws || ws_bytes < need)) return fail(KVB_ERR_WORKSPACE, "kvb_qkv_proj workspace too small");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  if (desc->dtype == KVB_BF16)
    return qkv_impl<bf16_t>(st, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v, ws);
  return qkv_impl<float>(st, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v, ws);
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
  if (!ws || ws_bytes < ws_mlp_bytes(desc, T_max)) return fail(KVB_ERR_WORKSPACE, "kvb_mlp workspace too small");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  if (desc->dtype == KVB_BF16)
    return mlp_impl<bf16_t>(st, desc, T_max, n_rows, row_tok, attn_o, w_o, hidden, norm2_w, w_gate_up, w_down, ws);
  return mlp_impl<float>(st, desc, T_max, n_rows, row_tok, attn_o, w_o, hidden, norm2_w, w_gate_up, w_down, ws);
}
