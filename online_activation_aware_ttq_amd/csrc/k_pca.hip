// Low-rank factors by PCA ("TTQ: Activation-Aware Test-Time Quantization
// ...": nl summary, Sec. 2, static factors initialised by PCA with dynamic
// adaptation supported; it summary, Sec. 2, B and A static or adapted online
// by PCA; zh summary, Sec. 2.2).  B (d' x r) is an orthonormal basis of the
// top-r left principal subspace of M = W (or M = W D^{1/2}, D from the
// current activations), A = B^T W, and the residual W - B A is what the
// quantizer sees.  The subspace comes from randomized subspace iteration
// (Halko, Martinsson and Tropp, 2011): Q = orth(M Omega), then per power
// iteration Z = orth(M^T Q), Q = orth(M Z); orth is CholeskyQR (Gram
// matrix, Cholesky in float64, Q = Y R^{-1}), twice for the final basis.
//
// Kernels (all float32 accumulation on the VALU: the products are skinny,
// r <= 128 columns, and the factors must be accurate to float32 before the
// final bf16 rounding):
//   k_skinny        one 64-row tile of C = A_s Bm over a K slice (split-K
//                   partials); A is W (bf16) or a float32 panel, read either
//                   row-wise (C = A Bm) or column-wise (C = A^T Bm); its
//                   columns may be scaled by D^{1/2} as they are staged
//   k_psum          ordered sum of the partials -> float32, and optionally
//                   bf16 (as is, or transposed)
//   k_cholinv       r <= 64: R^{-1} of the Gram matrix's Cholesky factor in
//                   one workgroup (float64 registers); Q = Y R^{-1} is then
//                   one more skinny product
//   k_chol, k_trsm  r = 128: Cholesky in one workgroup (float64 in LDS) and
//                   Q = Y R^{-1} by forward substitution, one row per lane
//   k_lr_residual   W_res = bf16(W - B A) from the bf16 factors
#include "ttq_internal.h"

namespace ttq {

namespace {

constexpr int SK_T = 64;  // rows of a C tile, and channels of a K tile

// a lane owns RW rows x CW columns of the 64 x N tile: (64 / RW) row groups
// times (N / CW) column groups = 256 lanes; within a wave the A values are a
// few contiguous LDS addresses and the Bm values a few broadcast ones
template <int N>
struct SkinnyShape {
  static constexpr int RW = N >= 16 ? 4 : 2;
  static constexpr int CW = N * RW >= 64 ? N * RW / 64 : 1;
};

template <int N, bool TN, typename TA>
__global__ __launch_bounds__(256) void k_skinny(SkinnyArgs a) {
  constexpr int RW = SkinnyShape<N>::RW, CW = SkinnyShape<N>::CW;
  constexpr int NRG = SK_T / RW;
  static_assert(NRG * (N / CW) == 256, "lane layout");
  __shared__ __attribute__((aligned(16))) float tA[SK_T][SK_T + 4];  // [k][row]
  __shared__ __attribute__((aligned(16))) float tB[SK_T][N];
  const int t = threadIdx.x;
  const int rg = t % NRG, cg = t / NRG;
  const int64_t r0 = (int64_t)blockIdx.x * SK_T;
  const int64_t k0 = (int64_t)blockIdx.y * a.kc;
  const int64_t k1 = min(a.K, k0 + a.kc);
  const TA* A = static_cast<const TA*>(a.A);
  // N >= 16: float32 matrix instructions, wave w owning rows 16w..16w+15 of
  // the tile and all N / 16 column blocks; N = 8: VALU FMAs, RW x CW per lane
  constexpr bool MF = N >= 16;
  constexpr int NCB = MF ? N / 16 : 1;
  const int lane = t & 63, wv = t >> 6;
  f32x4 macc[NCB];
  float acc[RW][CW];
#pragma unroll
  for (int c = 0; c < NCB; ++c) macc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[i][c] = 0.f;
  for (int64_t kt = k0; kt < k1; kt += SK_T) {
    // stage the A tile as [k][row]; element (row, k) is A[row][k] (C = A Bm)
    // or A[k][row] (C = A^T Bm); the index along the memory row is the one
    // the column scale applies to
    // a full tile with 16-byte aligned lines is read in 16-byte vectors along
    // the memory row; any other tile element by element
    const bool vec_a = kt + SK_T <= k1 && r0 + SK_T <= a.rows &&
                       a.lda % (int64_t)(16 / sizeof(TA)) == 0 &&
                       (reinterpret_cast<uintptr_t>(A) & 15) == 0;
    if (vec_a) {
      constexpr int VE = 16 / sizeof(TA), VPL = SK_T / VE;
#pragma unroll
      for (int p = 0; p < SK_T * VPL / 256; ++p) {
        const int vi = t + 256 * p;
        const int ln = vi / VPL, o = (vi % VPL) * VE;  // line, offset along it
        const int64_t off = TN ? (kt + ln) * a.lda + r0 + o : (r0 + ln) * a.lda + kt + o;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(A + off);
        float v[VE];
        if constexpr (sizeof(TA) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(raw[e] << 16);
            v[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(raw[e]);
        }
        if (a.scale) {
          const int64_t c0 = TN ? r0 + o : kt + o;
#pragma unroll
          for (int e = 0; e < VE; ++e) v[e] = v[e] * a.scale[c0 + e];
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          if (TN) tA[ln][o + e] = v[e];
          else tA[o + e][ln] = v[e];
        }
      }
    } else
    for (int e = t; e < SK_T * SK_T; e += 256) {
      int kk, rr;
      if (TN) { rr = e & 63; kk = e >> 6; }
      else { kk = e & 63; rr = e >> 6; }
      const int64_t row = r0 + rr, k = kt + kk;
      float v = 0.f;
      if (row < a.rows && k < k1) {
        const int64_t col = TN ? row : k;
        const int64_t off = TN ? k * a.lda + row : row * a.lda + k;
        if constexpr (sizeof(TA) == 2)
          v = __uint_as_float((unsigned)reinterpret_cast<const uint16_t*>(A)[off] << 16);
        else
          v = A[off];
        if (a.scale) v = v * a.scale[col];
      }
      tA[kk][rr] = v;
    }
    if (kt + SK_T <= k1 && a.ldb % 4 == 0 && (reinterpret_cast<uintptr_t>(a.Bm) & 15) == 0) {
      for (int vi = t; vi < SK_T * N / 4; vi += 256) {
        const int kk = vi / (N / 4), c0 = (vi % (N / 4)) * 4;
        *reinterpret_cast<f32x4*>(&tB[kk][c0]) =
            *reinterpret_cast<const f32x4*>(a.Bm + (kt + kk) * a.ldb + c0);
      }
    } else
    for (int e = t; e < SK_T * N; e += 256) {
      const int kk = e / N, c = e % N;
      const int64_t k = kt + kk;
      tB[kk][c] = k < k1 ? a.Bm[k * a.ldb + c] : 0.f;
    }
    __syncthreads();
    if constexpr (MF) {
      // 16x16x4 operands: lane (i, q) = (lane % 16, lane / 16) supplies
      // A[row i][k q] and Bm[k q][column i]
      const int i = lane & 15, q = lane >> 4;
#pragma unroll 4
      for (int k4 = 0; k4 < SK_T; k4 += 4) {
        const float af = tA[k4 + q][wv * 16 + i];
#pragma unroll
        for (int c = 0; c < NCB; ++c)
          macc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(af, tB[k4 + q][c * 16 + i],
                                                         macc[c], 0, 0, 0);
      }
      __syncthreads();
      continue;
    }
#pragma unroll 2
    for (int kk = 0; kk < SK_T; ++kk) {
      float av[RW], bv[CW];
#pragma unroll
      for (int i = 0; i < RW; ++i) av[i] = tA[kk][rg * RW + i];
#pragma unroll
      for (int c = 0; c < CW; ++c) bv[c] = tB[kk][cg * CW + c];
#pragma unroll
      for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[i][c] = fmaf(av[i], bv[c], acc[i][c]);
    }
    __syncthreads();
  }
  if constexpr (MF) {
    // result element (4 (lane / 16) + v, lane % 16) of each 16 x 16 block
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = r0 + wv * 16 + 4 * (lane >> 4) + v;
      if (row < a.rows) {
        float* out = a.part + ((int64_t)blockIdx.y * a.rows + row) * N + (lane & 15);
#pragma unroll
        for (int c = 0; c < NCB; ++c) out[c * 16] = macc[c][v];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int64_t row = r0 + rg * RW + i;
    if (row < a.rows) {
      float* out = a.part + ((int64_t)blockIdx.y * a.rows + row) * N + cg * CW;
#pragma unroll
      for (int c = 0; c < CW; ++c) out[c] = acc[i][c];
    }
  }
}

__global__ __launch_bounds__(256) void k_psum(PsumArgs a) {
  const int64_t total = a.rows * a.n;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    float v = 0.f;
#pragma unroll 8
    for (int z = 0; z < a.nsplit; ++z) v += a.part[(int64_t)z * total + e];
    if (a.out) a.out[e] = v;
    const int64_t i = e / a.n, c = e % a.n;
    if (a.out_bf16) a.out_bf16[e] = (bf16_t)f2bf(v);
    if (a.out_bf16_t) a.out_bf16_t[c * a.rows + i] = (bf16_t)f2bf(v);
  }
}

// A Gram pivot at or below this fraction of the largest diagonal entry is
// numerical noise (G is summed in float32: its relative rounding is about
// 1e-5 for the longest panels): the column carries no direction of its own.
// It is dropped -- its column of L, and its row and column of R^{-1}, are
// zero, so that column of Q = Y R^{-1} is zero and no other column depends on
// it -- and flagged, so that the final basis can be completed.  (Eliminating
// with such a pivot would amplify rounding noise by 1/sqrt(pivot) and can
// overflow.)
constexpr double kPivotDropTol = 1e-5;

// G (n x n, float32, symmetric up to rounding) -> R with G = R^T R, R upper
// triangular with a positive diagonal, Cholesky in float64 (right-looking,
// one barrier per step: row k is kept unscaled while the trailing matrix is
// updated with L[k][i] L[k][j] / pivot, and every row is scaled by 1/sqrt of
// its pivot at the end).  A pivot at or below kPivotDropTol of the largest
// diagonal entry drops its column (row k of R and R[k][k] are zero) and,
// when `defic` is given, is flagged there (1 for a dropped column, else 0).
// LDS rows have an odd stride n + 1.
__global__ __launch_bounds__(256) void k_chol(const float* G, float* R, int n,
                                              int* defic) {
  extern __shared__ double L[];  // n rows of n + 1, then the n pivots
  const int ld = n + 1;
  double* piv = L + n * ld;
  __shared__ double dmax;
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  for (int e = t; e < n * n; e += 256) {
    const int i = e / n, j = e % n;
    L[i * ld + j] = 0.5 * ((double)G[i * n + j] + (double)G[j * n + i]);
  }
  __syncthreads();
  if (t == 0) {
    double m = 0.0;
    for (int i = 0; i < n; ++i) m = fmax(m, L[i * ld + i]);
    dmax = m > 0.0 ? m : 1.0;
  }
  __syncthreads();
  const double tol = kPivotDropTol * dmax;
  for (int k = 0; k < n; ++k) {
    const double raw = L[k * ld + k];
    const bool drop = !(raw > tol);
    if (t == 0) {
      piv[k] = drop ? 0.0 : raw;
      if (defic) defic[k] = drop ? 1 : 0;
    }
    const double inv = drop ? 0.0 : 1.0 / raw;
    // row k does not change in step k: this lane's entries of it go to
    // registers, and each row's reads are issued before its writes (n - k - 1
    // <= 127 columns: 8 per lane cover them)
    double uk[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = k + 1 + tx + 16 * q;
      uk[q] = j < n ? L[k * ld + j] : 0.0;
    }
    for (int i = k + 1 + ty; i < n; i += 16) {
      const double lki = L[k * ld + i] * inv;
      double v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = k + 1 + tx + 16 * q;
        v[q] = (j < n && j >= i) ? L[i * ld + j] : 0.0;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = k + 1 + tx + 16 * q;
        if (j < n && j >= i) L[i * ld + j] = v[q] - lki * uk[q];
      }
    }
    __syncthreads();
  }
  for (int e = t; e < n * n; e += 256) {
    const int i = e / n, j = e % n;
    R[e] = piv[i] > 0.0 && i <= j
               ? (i < j ? (float)(L[i * ld + j] / sqrt(piv[i])) : (float)sqrt(piv[i]))
               : 0.f;
  }
}

// n <= 64: Cholesky and inverse in one workgroup of four waves, the rows in
// float64 registers.  Lane i of wave w holds the entries j = w (mod 4) of row
// i of G.  Step k (unrolled): in the wave holding column k the pivot comes
// from lane k (readlane) and every lane writes its L[i][k] to LDS; after one
// barrier every lane reads the column back as broadcasts and updates its
// entries of its row:
//   L[i][k] = g_i[k] / sqrt(p_k),  g_i[j] -= L[i][k] L[j][k]  (j > k)
// with 1/sqrt(p_k) from a Newton-refined estimate.
// Then every lane writes its entries of L to LDS as columns of L^T, and lane
// j of the first wave solves column j of L^{-1} in column order (column i of
// L read as broadcasts), starting from z = e_j:
//   z_i *= 1 / L[i][i],  z_m -= L[m][i] z_i  (m > i)
// so the updates of one step are independent of each other, and writes row
// j of R^{-1} = (L^{-1})^T: Rinv[j][i] = z_i.  (Splitting this solve over
// the four waves as well, with one barrier per step, measured no faster.)
__device__ __forceinline__ double bcast(double v, int lane) {
  const unsigned long long b = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)b, lane);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)(b >> 32), lane);
  return __longlong_as_double(((unsigned long long)hi << 32) | lo);
}

// 1/sqrt(p) for p > 0: the hardware estimate refined by two Newton steps
// y <- y (3/2 - (p/2) y^2), each of which roughly doubles the correct bits
__device__ __forceinline__ double rsqrt_f64(double p) {
  const double h = 0.5 * p;
  double y = __builtin_amdgcn_rsq(p);
  y = y * fma(-h * y, y, 1.5);
  y = y * fma(-h * y, y, 1.5);
  return y;
}

template <int N>
__global__ __launch_bounds__(256) void k_cholinv(const float* G, float* Rinv,
                                                 int* defic) {
  constexpr int NQ = N / 4;
  __shared__ double col[2][64];    // step k broadcasts through col[k & 1]
  __shared__ double Lt[N][N + 2];  // Lt[i][m] = L[m][i]
  __shared__ double dinv[N];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const bool live = l < N;
  double g[NQ];  // g[q] = G[l][w + 4 q], then L[l][w + 4 q]
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int j = w + 4 * q;
    g[q] = live ? 0.5 * ((double)G[l * N + j] + (double)G[j * N + l]) : 0.0;
  }
  // pivots at or below kPivotDropTol of the largest diagonal entry drop
  // their column
  double dmax = live ? (double)G[l * N + l] : 0.0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dmax = fmax(dmax, __shfl_xor(dmax, off));
  const double tol = kPivotDropTol * (dmax > 0.0 ? dmax : 1.0);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    if (w == (k & 3)) {  // the wave holding column k
      const double raw = bcast(g[k >> 2], k);
      const bool drop = !(raw > tol);
      if (defic && l == 0) defic[k] = drop ? 1 : 0;
      const double ir = drop ? 0.0 : rsqrt_f64(raw);
      const double lik = (l == k) ? raw * ir : g[k >> 2] * ir;
      g[k >> 2] = lik;  // L[l][k] (meaningful for l >= k)
      col[k & 1][l] = lik;
      if (l == 0) dinv[k] = ir;
    }
    // the barrier also retires step k - 1's reads of the other buffer
    // before step k + 1 overwrites it
    __syncthreads();
    const double lik = col[k & 1][l];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (w + 4 * q > k) g[q] = fma(-lik, col[k & 1][w + 4 * q], g[q]);
  }
  if (live) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) Lt[w + 4 * q][l] = g[q];
  }
  __syncthreads();
  if (w != 0) return;
  double z[N];
#pragma unroll
  for (int i = 0; i < N; ++i) z[i] = (i == l) ? 1.0 : 0.0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    z[i] *= dinv[i];
#pragma unroll
    for (int m = i + 1; m < N; ++m) z[m] = fma(-Lt[i][m], z[i], z[m]);
  }
  if (live) {
#pragma unroll
    for (int i = 0; i < N; ++i) Rinv[l * N + i] = (float)z[i];
  }
}

// Completion of a basis whose Gram matrix had dropped pivots (a panel of
// rank below n, e.g. from an all-zero M): each flagged column k of V
// [m][n] is replaced by a pseudo-random column of entries +-1/sqrt(m) (signs
// from a counter-based hash of (row, k)), which the next CholeskyQR pass
// orthonormalises against the others.  Unflagged columns are not touched, so
// a full-rank panel passes through unchanged.
__device__ __forceinline__ uint32_t hash_rc(uint32_t i, uint32_t k) {
  uint32_t h = i * 0x9E3779B1u ^ (k + 0x7F4A7C15u) * 0x85EBCA77u;
  h ^= h >> 16; h *= 0x7FEB352Du;
  h ^= h >> 15; h *= 0x846CA68Bu;
  h ^= h >> 16;
  return h;
}
__global__ __launch_bounds__(256) void k_pca_complete(float* V, int64_t m, int n,
                                                      const int* defic) {
  __shared__ int flag[128];
  const int t = threadIdx.x;
  const int f = t < n ? defic[t] : 0;
  if (t < n) flag[t] = f;
  if (!__syncthreads_or(f)) return;   // full-rank panel: nothing to do
  const int64_t i = (int64_t)blockIdx.x * 256 + t;
  if (i >= m) return;
  const float sc = 1.0f / sqrtf((float)m);
  for (int k = 0; k < n; ++k)
    if (flag[k]) V[i * n + k] = (hash_rc((uint32_t)i, (uint32_t)k) & 1u) ? sc : -sc;
}

// Q = Y R^{-1} in place, one row of Y per thread by forward substitution:
//   q_c = (y_c - sum_{m<c} q_m R[m][c]) / R[c][c]
// R is staged transposed (row c holds column c of R, its diagonal entry
// replaced by the reciprocal), so the terms of one q_c are contiguous and
// every lane reads the same addresses (broadcast).
template <int N>
__global__ __launch_bounds__(64) void k_trsm(float* Y, const float* R, int64_t m) {
  __shared__ __attribute__((aligned(16))) float sRt[N][N];
  const int t = threadIdx.x;
  for (int e = t; e < N * N; e += 64) {
    const int c = e / N, k = e % N;  // sRt[c][k] = R[k][c]
    // a dropped column has R[c][c] = 0: its q_c is zero
    const float rd = R[k * N + c];
    sRt[c][k] = c == k ? (rd > 0.f ? 1.0f / rd : 0.f) : (k < c ? rd : 0.f);
  }
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * 64 + t;
  if (i >= m) return;
  float q[N];
  float* row = Y + i * N;
#pragma unroll
  for (int c = 0; c < N; c += 4) {
    const f32x4 v = *(const f32x4*)(row + c);
    q[c] = v.x; q[c + 1] = v.y; q[c + 2] = v.z; q[c + 3] = v.w;
  }
#pragma unroll
  for (int c = 0; c < N; ++c) {
    float v = q[c];
#pragma unroll
    for (int k = 0; k < c; ++k) v = fmaf(-q[k], sRt[c][k], v);
    q[c] = v * sRt[c][c];
  }
#pragma unroll
  for (int c = 0; c < N; c += 4) *(f32x4*)(row + c) = f32x4{q[c], q[c + 1], q[c + 2], q[c + 3]};
}

// W_res[i][j] = bf16(W[i][j] - sum_c B[i][c] A[c][j]), a tile of 64 rows
// (32 for r = 128) x 64 columns per workgroup, float32 sums in c order.  A
// lane owns RT/16 rows x 4 columns; B is staged transposed so that a lane's
// rows and columns are each one contiguous LDS read per c.
template <int N>
constexpr int lr_rows() { return N >= 128 ? 32 : 64; }  // 64 KiB of static LDS

template <int N>
__global__ __launch_bounds__(256) void k_lr_residual(LrResidualArgs a) {
  constexpr int RT = lr_rows<N>();
  constexpr int RPT = RT / 16;  // rows per lane
  __shared__ __attribute__((aligned(16))) float sBt[N][RT];    // [c][row]
  __shared__ __attribute__((aligned(16))) float sA[N][SK_T];   // [c][col]
  const int t = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.y * RT, j0 = (int64_t)blockIdx.x * SK_T;
  for (int e = t; e < RT * N; e += 256) {
    const int rr = e / N, c = e % N;
    const int64_t i = i0 + rr;
    sBt[c][rr] = i < a.d_out ? bf16lo(a.B[i * N + c]) : 0.f;
  }
  for (int e = t; e < N * SK_T; e += 256) {
    const int c = e / SK_T, jj = e % SK_T;
    const int64_t j = j0 + jj;
    sA[c][jj] = j < a.d ? bf16lo(a.A[(int64_t)c * a.d + j]) : 0.f;
  }
  __syncthreads();
  const int rq = t / 16, cq = t % 16;
  float acc[RPT][4];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[r][q] = 0.f;
#pragma unroll 4
  for (int c = 0; c < N; ++c) {
    float bv[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) bv[r] = sBt[c][rq * RPT + r];
    const f32x4 av = *(const f32x4*)&sA[c][cq * 4];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      acc[r][0] = fmaf(bv[r], av.x, acc[r][0]);
      acc[r][1] = fmaf(bv[r], av.y, acc[r][1]);
      acc[r][2] = fmaf(bv[r], av.z, acc[r][2]);
      acc[r][3] = fmaf(bv[r], av.w, acc[r][3]);
    }
  }
  // a lane's 4 columns as one 8-byte load of W and store of W_res where the
  // row is aligned for it, element by element otherwise
  const int64_t jv = j0 + cq * 4;
  const bool vec = jv + 4 <= a.d && (a.d & 3) == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.W) | reinterpret_cast<uintptr_t>(a.Wres)) & 7) == 0;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int64_t i = i0 + rq * RPT + r;
    if (i >= a.d_out) break;
    if (vec) {
      const u32x2 wv = *reinterpret_cast<const u32x2*>(a.W + i * a.d + jv);
      const float w0 = __uint_as_float(wv.x << 16), w1 = __uint_as_float(wv.x & 0xffff0000u);
      const float w2 = __uint_as_float(wv.y << 16), w3 = __uint_as_float(wv.y & 0xffff0000u);
      u32x2 o;
      o.x = (f2bf(w0 - acc[r][0]) & 0xffffu) | (f2bf(w1 - acc[r][1]) << 16);
      o.y = (f2bf(w2 - acc[r][2]) & 0xffffu) | (f2bf(w3 - acc[r][3]) << 16);
      *reinterpret_cast<u32x2*>(a.Wres + i * a.d + jv) = o;
      continue;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t j = j0 + cq * 4 + q;
      if (j < a.d) {
        const float w = bf16lo(a.W[i * a.d + j]);
        a.Wres[i * a.d + j] = (bf16_t)f2bf(w - acc[r][q]);
      }
    }
  }
}

template <bool TN, typename TA>
hipError_t launch_skinny_t(const SkinnyArgs& a, dim3 grid, const Launch& L) {
  switch (a.n) {
    case 8: return ext_launch(k_skinny<8, TN, TA>, grid, dim3(256), 0, L, a);
    case 16: return ext_launch(k_skinny<16, TN, TA>, grid, dim3(256), 0, L, a);
    case 32: return ext_launch(k_skinny<32, TN, TA>, grid, dim3(256), 0, L, a);
    case 64: return ext_launch(k_skinny<64, TN, TA>, grid, dim3(256), 0, L, a);
    case 128: return ext_launch(k_skinny<128, TN, TA>, grid, dim3(256), 0, L, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int skinny_splits(int64_t rows, int64_t K) {
  // about 1536 workgroups (six per CU) so that the loads of one hide behind
  // the arithmetic of the others
  const int64_t tiles = (rows + SK_T - 1) / SK_T;
  int64_t s = (1536 + tiles - 1) / tiles;
  // at least 256 channels a split, but one K tile for the small products
  // (the r x r Gram matrices: one or two row tiles)
  const int64_t smax = tiles <= 2 ? (K + SK_T - 1) / SK_T : (K + 255) / 256;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  // whole K tiles per split
  const int64_t kc = ((K + s - 1) / s + SK_T - 1) / SK_T * SK_T;
  return (int)((K + kc - 1) / kc);
}

int64_t skinny_kc(int64_t K, int splits) {
  return ((K + splits - 1) / splits + SK_T - 1) / SK_T * SK_T;
}

hipError_t launch_skinny(const SkinnyArgs& a, bool tn, bool a_bf16, const Launch& L) {
  if (a.rows <= 0 || a.K <= 0) return hipSuccess;
  if (a.kc <= 0 || a.kc % SK_T != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.rows + SK_T - 1) / SK_T), (unsigned)((a.K + a.kc - 1) / a.kc));
  if (tn) return a_bf16 ? launch_skinny_t<true, bf16_t>(a, grid, L)
                        : launch_skinny_t<true, float>(a, grid, L);
  return a_bf16 ? launch_skinny_t<false, bf16_t>(a, grid, L)
                : launch_skinny_t<false, float>(a, grid, L);
}

hipError_t launch_psum(const PsumArgs& a, const Launch& L) {
  const int64_t total = a.rows * a.n;
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  return ext_launch(k_psum, dim3((unsigned)blocks), dim3(256), 0, L, a);
}

hipError_t launch_pca_complete(float* V, int64_t m, int n, const int* defic,
                               const Launch& L) {
  if (m <= 0 || n <= 0 || n > 128) return m <= 0 ? hipSuccess : hipErrorInvalidValue;
  return ext_launch(k_pca_complete, dim3((unsigned)((m + 255) / 256)), dim3(256), 0,
                    L, V, m, n, defic);
}

hipError_t launch_chol(const float* G, float* R, int n, int* defic,
                       const Launch& L) {
  if (n <= 0 || n > 128) return hipErrorInvalidValue;
  const uint32_t lds = (uint32_t)((n * (n + 1) + n) * sizeof(double));
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(k_chol),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)((128 * 129 + 128) * sizeof(double)));
  if (attr != hipSuccess) return attr;
  return ext_launch(k_chol, dim3(1), dim3(256), lds, L, G, R, n, defic);
}

hipError_t launch_cholinv(const float* G, float* Rinv, int n, int* defic,
                          const Launch& L) {
  switch (n) {
    case 8: return ext_launch(k_cholinv<8>, dim3(1), dim3(256), 0, L, G, Rinv, defic);
    case 16: return ext_launch(k_cholinv<16>, dim3(1), dim3(256), 0, L, G, Rinv, defic);
    case 32: return ext_launch(k_cholinv<32>, dim3(1), dim3(256), 0, L, G, Rinv, defic);
    case 64: return ext_launch(k_cholinv<64>, dim3(1), dim3(256), 0, L, G, Rinv, defic);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_trsm(float* Y, const float* R, int64_t m, int n, const Launch& L) {
  if (m <= 0) return hipSuccess;
  const dim3 grid((unsigned)((m + 63) / 64));
  switch (n) {
    case 8: return ext_launch(k_trsm<8>, grid, dim3(64), 0, L, Y, R, m);
    case 16: return ext_launch(k_trsm<16>, grid, dim3(64), 0, L, Y, R, m);
    case 32: return ext_launch(k_trsm<32>, grid, dim3(64), 0, L, Y, R, m);
    case 64: return ext_launch(k_trsm<64>, grid, dim3(64), 0, L, Y, R, m);
    case 128: return ext_launch(k_trsm<128>, grid, dim3(64), 0, L, Y, R, m);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lr_residual(const LrResidualArgs& a, int n, const Launch& L) {
  if (a.d_out <= 0 || a.d <= 0) return hipSuccess;
  const unsigned gx = (unsigned)((a.d + SK_T - 1) / SK_T);
#define TTQ_LR_CASE(NV)                                                        \
  case NV:                                                                     \
    return ext_launch(k_lr_residual<NV>,                                       \
                      dim3(gx, (unsigned)((a.d_out + lr_rows<NV>() - 1) /      \
                                          lr_rows<NV>())),                     \
                      dim3(256), 0, L, a);
  switch (n) {
    TTQ_LR_CASE(8)
    TTQ_LR_CASE(16)
    TTQ_LR_CASE(32)
    TTQ_LR_CASE(64)
    TTQ_LR_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef TTQ_LR_CASE
}

}  // namespace ttq
