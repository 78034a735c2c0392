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
// TM x TN tiles of v_mfma_f32_32x32x16_bf16; block tile BM = 64 TM, BN = 64 TN
// rows of B.  K advances in 64-wide steps through double-buffered LDS (row
// stride 72 elements: conflict-free 16-byte fragment reads); the next step's
// tiles are fetched into registers while the current one feeds the MFMAs.
//
// SwiGLU (DUAL): the B tile interleaves 32-row subtiles of the gate and up
// matrices (gate cols c..c+31, up cols c..c+31, ...), so a wave holds gate
// and up of the same outputs in neighbouring accumulators; BN/2 outputs wide.

constexpr int BK = 64, LDK = BK + 8;  // LDS row stride in bf16 elements
constexpr int GEMM_THREADS = 256;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// multiply 8 bf16 by 8 bf16 gains, round back to bf16
__device__ __forceinline__ uint4 mul_gain(const uint4& a, const uint4& g) {
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, gw[4] = {g.x, g.y, g.z, g.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float lo = __uint_as_float(aw[i] << 16) * __uint_as_float(gw[i] << 16);
    const float hi = __uint_as_float(aw[i] & 0xffff0000u) * __uint_as_float(gw[i] & 0xffff0000u);
    o[i] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float sumsq8(const uint4& a) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
    s += lo * lo;
    s += hi * hi;
  }
  return s;
}

template <int TM, int TN>
struct Tile {
  static constexpr int BM = 64 * TM, BN = 64 * TN;
  static constexpr int A_LD = BM / 32, B_LD = BN / 32;  // 16-byte loads per thread per K step
  static constexpr size_t LDS = (size_t)2 * (BM + BN) * LDK * sizeof(bf16_t);
  // the epilogue reuses the same LDS for a [BM/2][OUT_N + 8] float tile
  static_assert((size_t)(BM / 2) * (BN + 8) * 4 <= LDS, "epilogue tile must fit the K-loop buffers");
};

template <int MODE, bool DUAL, bool NORM, bool GAIN, int TM, int TN>
__global__ void __launch_bounds__(GEMM_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bf16_kernel(GemmArgs<bf16_t> p) {
  using TL = Tile<TM, TN>;
  constexpr int BM = TL::BM, BN = TL::BN, A_LD = TL::A_LD, B_LD = TL::B_LD;
  constexpr int OUT_N = DUAL ? BN / 2 : BN;  // output columns per block
  extern __shared__ __align__(16) uint8_t smem[];
  bf16_t* sA = reinterpret_cast<bf16_t*>(smem);  // [2][BM][LDK]
  bf16_t* sB = sA + 2 * BM * LDK;                // [2][BN][LDK]
  __shared__ float s_rinv[NORM ? BM : 1];

  const int M = row_count(p.n_rows, p.M_max);
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * OUT_N;
  if (m0 >= M) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = (wave >> 1) * (32 * TM), wn = (wave & 1) * (32 * TN);

  // loaders: chunk c = t + 256 i -> tile row c / 8 = t / 8 + 32 i, k-chunk c % 8 = t % 8
  const int lrow = t >> 3, lkc = t & 7;
  const bf16_t* a_src[A_LD];
  const bf16_t* b_src[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; i++) {
    int m = m0 + lrow + 32 * i;
    m = m < M ? m : M - 1;
    const int ar = p.a_rows ? p.a_rows[m] : m;
    a_src[i] = p.A + (size_t)ar * p.K + lkc * 8;
  }
#pragma unroll
  for (int i = 0; i < B_LD; i++) {
    const int b = lrow + 32 * i;  // B-tile row; subtile b / 32 == i
    const bf16_t* base = p.B;
    int n;
    if (DUAL) {
      base = (i & 1) ? p.B2 : p.B;
      n = n0 + (i >> 1) * 32 + (b & 31);
    } else {
      n = n0 + b;
    }
    n = n < p.N ? n : p.N - 1;
    b_src[i] = base + (size_t)n * p.K + lkc * 8;
  }
  uint4 ra[A_LD], rb[B_LD];
  float ssq[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; i++) ssq[i] = 0.f;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = (f32x16_t){};

  const int KT = p.K / BK;
  // prologue: tile 0 -> LDS buffer 0
#pragma unroll
  for (int i = 0; i < A_LD; i++) ra[i] = *reinterpret_cast<const uint4*>(a_src[i]);
#pragma unroll
  for (int i = 0; i < B_LD; i++) rb[i] = *reinterpret_cast<const uint4*>(b_src[i]);
  {
    uint4 g = make_uint4(0, 0, 0, 0);
    if (GAIN) g = *reinterpret_cast<const uint4*>(p.norm_w + lkc * 8);
#pragma unroll
    for (int i = 0; i < A_LD; i++) {
      uint4 a = ra[i];
      if (NORM) ssq[i] += sumsq8(a);
      if (GAIN) a = mul_gain(a, g);
      *reinterpret_cast<uint4*>(sA + (lrow + 32 * i) * LDK + lkc * 8) = a;
    }
#pragma unroll
    for (int i = 0; i < B_LD; i++) *reinterpret_cast<uint4*>(sB + (lrow + 32 * i) * LDK + lkc * 8) = rb[i];
  }
  __syncthreads();

  const int fr = lane & 31, fk = (lane >> 5) * 8;  // fragment row, k offset in a 16-wide slice
  for (int kt = 0; kt < KT; kt++) {
    const int buf = kt & 1;
    // next K step (the last iteration re-fetches its own step; the copy is never read)
    const int kn = kt + 1 < KT ? kt + 1 : kt;
    {
      const int ko = kn * BK;
#pragma unroll
      for (int i = 0; i < A_LD; i++) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + ko);
#pragma unroll
      for (int i = 0; i < B_LD; i++) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + ko);
    }
    const bf16_t* a_s = sA + buf * BM * LDK + (wm + fr) * LDK + fk;
    const bf16_t* b_s = sB + buf * BN * LDK + (wn + fr) * LDK + fk;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; i++) af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(a_s + i * 32 * LDK + kk));
#pragma unroll
      for (int j = 0; j < TN; j++) bfr[j] = as_bf16x8(*reinterpret_cast<const uint4*>(b_s + j * 32 * LDK + kk));
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    {
      const int nb = buf ^ 1;
      const bool fresh = kt + 1 < KT;  // only a real next step adds to the row sums
      uint4 g = make_uint4(0, 0, 0, 0);
      if (GAIN) g = *reinterpret_cast<const uint4*>(p.norm_w + kn * BK + lkc * 8);
#pragma unroll
      for (int i = 0; i < A_LD; i++) {
        uint4 a = ra[i];
        if (NORM) ssq[i] += fresh ? sumsq8(a) : 0.f;
        if (GAIN) a = mul_gain(a, g);
        *reinterpret_cast<uint4*>(sA + (nb * BM + lrow + 32 * i) * LDK + lkc * 8) = a;
      }
#pragma unroll
      for (int i = 0; i < B_LD; i++)
        *reinterpret_cast<uint4*>(sB + (nb * BN + lrow + 32 * i) * LDK + lkc * 8) = rb[i];
    }
    __syncthreads();
  }

  if (NORM) {
#pragma unroll
    for (int i = 0; i < A_LD; i++) {
      float s = ssq[i];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if (lkc == 0) s_rinv[lrow + 32 * i] = 1.f / sqrtf(s / (float)p.K + p.eps);
    }
    __syncthreads();
  }

  // Epilogue, staged through LDS in two halves of BM/2 rows: the waves owning a
  // half write their float accumulators (SwiGLU already combined) to an
  // [BM/2][OUT_N] tile, then all threads read 8 consecutive outputs of a row,
  // apply the mode (scale, residual, scatter) and store 16 bytes at a time.
  // acc[i][j][r] sits at tile row wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,
  // tile col wn + 32 j + lane % 32 (DUAL: output col (wn / 32 + j) / 2 * 32 + lane % 32).
  constexpr int HR = BM / 2;
  constexpr int LDC = OUT_N + 8;  // floats; rows 4 apart land 32 banks apart
  float* sC = reinterpret_cast<float*>(smem);
  const int lc = lane & 31;
  const int my_half = wave >> 1;
#pragma unroll
  for (int half = 0; half < 2; half++) {
    if (my_half == half) {
#pragma unroll
      for (int j = 0; j < TN; j += (DUAL ? 2 : 1)) {
        const int cl = DUAL ? ((wn / 32 + j) >> 1) * 32 + lc : wn + j * 32 + lc;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int rl = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);  // row inside the half
            float v = acc[i][j][r];
            if (DUAL) {
              const float rinv = s_rinv[half * HR + rl];
              v = silu(v * rinv) * (acc[i][j + 1][r] * rinv);
            }
            sC[rl * LDC + cl] = v;
          }
      }
    }
    __syncthreads();
    constexpr int CPR = OUT_N / 8;  // 8-output chunks per row
    for (int c = t; c < HR * CPR; c += GEMM_THREADS) {
      const int rl = c / CPR, cc = (c % CPR) * 8;
      const int ml = half * HR + rl, m = m0 + ml, n = n0 + cc;
      if (m >= M || n >= p.N) continue;
      const float4 lo = *reinterpret_cast<const float4*>(sC + rl * LDC + cc);
      const float4 hi = *reinterpret_cast<const float4*>(sC + rl * LDC + cc + 4);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      bf16_t* dst;
      if (MODE == EPI_QKV) {
        const float rinv = s_rinv[ml];
#pragma unroll
        for (int e = 0; e < 8; e++) v[e] *= rinv;
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
      uint4 o;
      o.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
      o.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
      o.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
      o.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
      *reinterpret_cast<uint4*>(dst) = o;
    }
    __syncthreads();
  }
}

template <int MODE, bool DUAL, bool NORM, bool GAIN, int TM, int TN>
static kvb_status launch_bf16(hipStream_t st, const GemmArgs<bf16_t>& p, const char* name) {
  using TL = Tile<TM, TN>;
  constexpr int OUT_N = DUAL ? TL::BN / 2 : TL::BN;
  dim3 grid(cdiv(p.M_max, TL::BM), cdiv(p.N, OUT_N));
  static bool attr_set = false;  // opt in to > 64 KiB of dynamic LDS once per instantiation
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<MODE, DUAL, NORM, GAIN, TM, TN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)TL::LDS);
    if (e != hipSuccess) return fail(KVB_ERR_HIP, std::string("hipFuncSetAttribute: ") + hipGetErrorString(e));
    attr_set = true;
  }
  {
    LaunchTimer lt(st, name);
    gemm_bf16_kernel<MODE, DUAL, NORM, GAIN, TM, TN><<<grid, GEMM_THREADS, TL::LDS, st>>>(p);
  }
  return check_launch("gemm_bf16_kernel");
}

// Tile choice: the per-element reduction order (64-wide K steps, 16-wide MFMA
// slices in order) is the same for every tile shape, so picking the shape from
// the launch bound keeps every row's result independent of the batch.
template <int MODE, bool DUAL, bool NORM, bool GAIN>
static kvb_status run_bf16_g(hipStream_t st, const GemmArgs<bf16_t>& p, const char* name) {
  const Ctx* c = current_ctx();
  const long cus = c ? c->n_cu : 256;
  const long big_blocks = (long)cdiv(p.M_max, 256) * cdiv(p.N, DUAL ? 128 : 256);
  if (big_blocks >= cus) return launch_bf16<MODE, DUAL, NORM, GAIN, 4, 4>(st, p, name);
  const long mid_blocks = (long)cdiv(p.M_max, 256) * cdiv(p.N, DUAL ? 64 : 128);
  if (mid_blocks >= cus) return launch_bf16<MODE, DUAL, NORM, GAIN, 4, 2>(st, p, name);
  return launch_bf16<MODE, DUAL, NORM, GAIN, 2, 2>(st, p, name);
}

// Tile choice: the per-element reduction order (64-wide K steps, 16-wide MFMA
// slices in order) is the same for every tile shape, so picking the shape from
// the launch bound keeps every row's result independent of the batch.  RMSNorm
// gains are applied to A only when given (NULL = unit gains).
template <int MODE, bool DUAL, bool NORM>
static kvb_status run_bf16(hipStream_t st, const GemmArgs<bf16_t>& p, const char* name) {
  if (p.M_max == 0 || p.N == 0) return KVB_OK;
  if constexpr (NORM) {
    if (p.norm_w) return run_bf16_g<MODE, DUAL, NORM, true>(st, p, name);
  }
  return run_bf16_g<MODE, DUAL, NORM, false>(st, p, name);
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
                           const int32_t* tok_pos, void* q, void* k, void* v) {
  GemmArgs<T> p{};
  p.A = (const T*)hidden;
  p.a_rows = row_tok;
  p.B = (const T*)w_qkv;
  p.norm_w = (const T*)norm_w;
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
  if constexpr (sizeof(T) == 2) KVB_TRY((run_bf16<EPI_QKV, false, true>(st, p, "gemm_qkv")));
  else KVB_TRY((run_f32<EPI_QKV, false, true>(st, p, "gemm_qkv")));
  if (tok_pos) return launch_rope<T>(st, T_max, n_rows, row_tok, tok_pos, q, k, d);
  return KVB_OK;
}

template <class T>
static kvb_status mlp_impl(hipStream_t st, const kvb_model_desc* d, int T_max, const int32_t* n_rows,
                           const int32_t* row_tok, const void* attn_o, const void* w_o, void* hidden,
                           const void* norm2_w, const void* w_gate_up, const void* w_down, void* ws) {
  const int D = d->d_model, F = d->ffn, QD = d->n_q_heads * d->head_dim;
  T* h1 = (T*)ws;
  T* u = (T*)((char*)ws + align_up((size_t)T_max * D * sizeof(T), 256));
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
    KVB_TRY((run_bf16<EPI_RESID, false, false>(st, a, "gemm_oproj")));
    KVB_TRY((run_bf16<EPI_SWIGLU, true, true>(st, b, "gemm_swiglu")));
    return run_bf16<EPI_SCATTER, false, false>(st, c, "gemm_down");
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
                                   void* v) {
  KVB_TRY(check_ctx(ctx));
  KVB_TRY(check_desc(desc));
  if (T_max < 0) return fail(KVB_ERR_INVALID_ARG, "T_max < 0");
  if (T_max == 0) return KVB_OK;
  KVB_CHECK_PTR(hidden, "hidden");
  KVB_CHECK_PTR(w_qkv, "w_qkv");
  KVB_CHECK_PTR(q, "q");
  KVB_CHECK_PTR(k, "k");
  KVB_CHECK_PTR(v, "v");
  CtxScope scope(ctx);
  hipStream_t st = (hipStream_t)stream;
  if (desc->dtype == KVB_BF16)
    return qkv_impl<bf16_t>(st, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v);
  return qkv_impl<float>(st, desc, T_max, n_rows, row_tok, hidden, norm_w, w_qkv, tok_pos, q, k, v);
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
