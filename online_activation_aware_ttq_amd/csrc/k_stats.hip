// Activation statistics of the TTQ linear projection on gfx950.
//
// Per input channel i: n_i = ||X_{i,:}||_p over the tokens, then
// D^{1/2}_ii = (n_i + lambda)^{alpha/2} and D^{-1/2}_ii = 1 / D^{1/2}_ii
// ("TTQ: Activation-Aware Test-Time Quantization ...", gist.science zh
// summary, Sec. 2.1; the norm is not normalised by T, lambda is added to the
// norm before the power).  Sums and powers are evaluated in float64 -- the
// CDNA vector unit runs fp64 at the fp32 rate and this reduction is bound by
// the X read, so the extra precision is free -- and rounded once to fp32.
//
// X is token-major [T][d]; a lane owns 8 consecutive channels (one 16-byte
// load per token), so every load of a wave is a contiguous 1 KiB row piece.
#include "ttq_internal.h"

namespace ttq {

__device__ __forceinline__ double pow_term(float x, int pmode, double p) {
  double a = fabs((double)x);
  if (pmode == 2) return a * a;
  if (pmode == 1) return a;
  return a == 0.0 ? 0.0 : pow(a, p);
}

__device__ __forceinline__ double finish_norm(double S, int pmode, double p) {
  if (pmode == 2) return sqrt(S);
  if (pmode == 1) return S;
  return pow(S, 1.0 / p);
}

// (n + lambda)^{alpha/2} and its reciprocal; a channel with n + lambda == 0
// multiplies only zero activations and gets the neutral scale 1.
__device__ __forceinline__ void diag_half(double n, double lam, double alpha,
                                          float& dh, float& dhi) {
  double base = n + lam;
  double h = 1.0;
  if (base > 0.0) {
    // correctly rounded square roots for the common exponents, pow otherwise;
    // either is within ~1 ulp of float64 before the single fp32 rounding
    if (alpha == 0.5) h = sqrt(sqrt(base));
    else if (alpha == 1.0) h = sqrt(base);
    else if (alpha == 2.0) h = base;
    else if (alpha != 0.0) h = pow(base, 0.5 * alpha);
  }
  dh = (float)h;
  dhi = (float)(1.0 / h);
}

__device__ __forceinline__ void accum8(double acc[8], u32x4 v, int pmode,
                                       double p) {
  acc[0] += pow_term(bf16lo(v.x), pmode, p);
  acc[1] += pow_term(bf16hi(v.x), pmode, p);
  acc[2] += pow_term(bf16lo(v.y), pmode, p);
  acc[3] += pow_term(bf16hi(v.y), pmode, p);
  acc[4] += pow_term(bf16lo(v.z), pmode, p);
  acc[5] += pow_term(bf16hi(v.z), pmode, p);
  acc[6] += pow_term(bf16lo(v.w), pmode, p);
  acc[7] += pow_term(bf16hi(v.w), pmode, p);
}

// ---------------------------------------------------------------------------
// Small T (T <= 128, fused path and statistics-only calls): a workgroup of
// NT = 512 threads owns BC channels (128, or 256 for groups of 256: always whole
// quantization groups) and every token for the statistics, and writes x' for
// one 32-token slice (the slices' workgroups repeat the statistics: X is
// small, and the chip has more CUs than there are channel blocks).  Thread
// (token lane tl, channel chunk cq) loads the tokens tl + i * TLN of 8
// consecutive channels; the float64 partial powers are summed over the token
// lanes of a wave (fixed butterfly), then over the waves in LDS in order, one
// thread per channel finishes D^{+-1/2}.  Then the threads holding the
// slice's tokens write x' = x * D^{-1/2} (the fused kernels' MFMA operand)
// and the group sums of x' per token.
//
// For T <= 16 x' is carried as an unevaluated pair of bf16 numbers hi + lo
// (hi = bf16(x'), lo = bf16(x' - hi)), about 16 significant bits: with few
// tokens one outlier channel can dominate every output and a single bf16
// rounding of it would be shared by all of them.  For larger T a single bf16
// plane is written.  Planes are in MFMA fragment order (xs_frag_index) and
// zero-padded to whole 16-token blocks.  The group sums are of exactly the
// values written, zero past T up to the padded token count.
// ---------------------------------------------------------------------------
// (512 threads: measured on MI355X, one or two 16-token steps take about
// 1 us less than with 1024, whose extra token lanes sit idle for small T and
// add a deeper cross-wave reduction)
constexpr int kStatsThreads = 512;

template <int PM, int BC, int NT>
__global__ __launch_bounds__(NT) void k_stats_small(StatsSmallArgs a) {
  constexpr int NCH = BC / 8;          // channel chunks
  constexpr int TLN = NT / NCH;        // token lanes
  constexpr int TPW = 64 / NCH;        // token lanes per wave
  constexpr int NTK = 128 / TLN;       // tokens per thread (T <= 128)
  constexpr int NWV = NT / 64;         // waves
  __shared__ double red[NWV][BC];
  __shared__ float dhi_l[BC];
  const int tid = threadIdx.x;
  const int cq = tid % NCH, tl = tid / NCH;
  const int wv = tid >> 6;
  const int r = blockIdx.z;
  const int64_t c0 = (int64_t)blockIdx.x * BC + cq * 8;
  const bool live = c0 < a.d;
  const bf16_t* X = a.X + (int64_t)r * a.T * a.d;

  u32x4 v[NTK];
#pragma unroll
  for (int i = 0; i < NTK; ++i) {
    const int64_t t = tl + i * TLN;
    v[i] = (live && t < a.T) ? *(const u32x4*)(X + t * a.d + c0)
                             : u32x4{0u, 0u, 0u, 0u};
  }
  if (a.dhi_in) {
    // stored D^{-1/2}: no statistics
    if (tid < BC) {
      const int64_t c = (int64_t)blockIdx.x * BC + tid;
      dhi_l[tid] = c < a.d ? a.dhi_in[(int64_t)r * a.d + c] : 1.f;
    }
  } else {  // statistics (uniform branch)
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NTK; ++i)
      if (live && tl + i * TLN < a.T) accum8(acc, v[i], PM, a.p);
    // token lanes of this wave (lanes cq, cq + NCH, ...): fixed butterfly
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int off = NCH; off < 64; off <<= 1) acc[j] += __shfl_xor(acc[j], off);
      if (tl % TPW == 0) red[wv][cq * 8 + j] = acc[j];
    }
    __syncthreads();
    if (tid < BC) {
      const int64_t c = (int64_t)blockIdx.x * BC + tid;
      double S = 0.0;
#pragma unroll
      for (int k = 0; k < NWV; ++k) S += red[k][tid];
      float dh = 1.f, dhi = 1.f;
      if (c < a.d) {
        diag_half(finish_norm(S, PM, a.p), a.lam, a.alpha, dh, dhi);
        if (blockIdx.y == 0) {  // one of the token slices publishes
          a.dh[(int64_t)r * a.d + c] = dh;
          a.dhi[(int64_t)r * a.d + c] = dhi;
          if (a.dh_export) a.dh_export[(int64_t)r * a.d + c] = dh;
        }
      }
      dhi_l[tid] = dhi;
    }
  }
  if (!a.xs) return;
  __syncthreads();

  const bool tiled = a.planes == 1;
  const int ntb = a.Tp / 16;
  const int G = (int)(a.d / a.group);
  const int lpg = a.group >> 3;  // chunk lanes per quantization group
  bf16_t* xs = a.xs + (int64_t)r * (tiled ? 1 : 2) * a.Tp * a.d;
  bf16_t* xs_lo = xs + (int64_t)a.Tp * a.d;
  float* sx = a.sx + (int64_t)r * G * a.Tp;
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sc[j] = dhi_l[cq * 8 + j];
  // fragment of these 8 channels (see xs_frag_index): MFMA step and lane
  // quarter, in step-major or quarter order
  const int64_t g = c0 / a.group, cig = c0 % a.group;
  const int64_t k = a.quarter ? (cig % (a.group / 4)) / 8 : cig / 32;
  const int lane_q = (int)(a.quarter ? cig / (a.group / 4) : (cig % 32) / 8) * 16;
#pragma unroll
  for (int i = 0; i < NTK; ++i) {
    const int64_t t = tl + i * TLN;
    if (t >= a.Tp) break;  // uniform across the chunk lanes of a token
    if ((t >> 5) != (int64_t)blockIdx.y) continue;  // another slice's token
    float ps = 0.f;
    u32x4 o = {0u, 0u, 0u, 0u}, ol = {0u, 0u, 0u, 0u};
    if (live && t < a.T) {
      const float x[8] = {bf16lo(v[i].x), bf16hi(v[i].x), bf16lo(v[i].y),
                          bf16hi(v[i].y), bf16lo(v[i].z), bf16hi(v[i].z),
                          bf16lo(v[i].w), bf16hi(v[i].w)};
      unsigned bh[8], bl[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xp = x[j] * sc[j];
        bh[j] = f2bf(xp);
        const float hi = __uint_as_float(bh[j] << 16);
        bl[j] = f2bf(xp - hi);
        ps += tiled ? hi : hi + __uint_as_float(bl[j] << 16);
      }
      o = u32x4{bh[0] | (bh[1] << 16), bh[2] | (bh[3] << 16),
                bh[4] | (bh[5] << 16), bh[6] | (bh[7] << 16)};
      ol = u32x4{bl[0] | (bl[1] << 16), bl[2] | (bl[3] << 16),
                 bl[4] | (bl[5] << 16), bl[6] | (bl[7] << 16)};
    }
    if (live) {
      const int lane = lane_q + (int)(t & 15);
      const int64_t fi = 8 * xs_frag_index(g, t >> 4, k, lane, ntb, a.group);
      *(u32x4*)(xs + fi) = o;
      if (!tiled) *(u32x4*)(xs_lo + fi) = ol;
    }
    // the chunk lanes of one group are adjacent within a token row
    for (int off = lpg >> 1; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    if (live && (cq % lpg) == 0) sx[g * a.Tp + t] = ps;
  }
}

hipError_t launch_stats_small(const StatsSmallArgs& a, int R, const Launch& L) {
  if (a.T > 128) return hipErrorInvalidValue;
  // x' of 32-token slices in separate workgroups (each takes the statistics
  // of all tokens itself; one of them publishes D^{+-1/2})
  const unsigned nsl = a.xs ? (unsigned)((a.Tp + 31) / 32) : 1u;
  const dim3 blk(kStatsThreads);
  if (a.group == 256) {
    const dim3 grid((unsigned)((a.d + 255) / 256), nsl, (unsigned)R);
    if (a.pmode == 2) return ext_launch(k_stats_small<2, 256, kStatsThreads>, grid, blk, 0, L, a);
    if (a.pmode == 1) return ext_launch(k_stats_small<1, 256, kStatsThreads>, grid, blk, 0, L, a);
    return ext_launch(k_stats_small<0, 256, kStatsThreads>, grid, blk, 0, L, a);
  }
  const dim3 grid((unsigned)((a.d + 127) / 128), nsl, (unsigned)R);
  if (a.pmode == 2) return ext_launch(k_stats_small<2, 128, kStatsThreads>, grid, blk, 0, L, a);
  if (a.pmode == 1) return ext_launch(k_stats_small<1, 128, kStatsThreads>, grid, blk, 0, L, a);
  return ext_launch(k_stats_small<0, 128, kStatsThreads>, grid, blk, 0, L, a);
}

// ---------------------------------------------------------------------------
// Large T: each wave reduces one slice of tokens for 512 channels; the four
// waves of a block add their slices in LDS in slice order and write one
// float64 partial per block; a finalize pass sums the block partials in
// order (deterministic).
// ---------------------------------------------------------------------------
// The p mode is a template parameter: with the general-p branch in the loop
// the kernel needs 160 VGPRs (3 waves per SIMD) and streamed X at about
// 3.8 TB/s; the p = 2 instantiation (54 VGPRs) reads it at 5.8 TB/s, against
// 7.2 TB/s for a plain read kernel (8 requests x 4096 tokens x 4096
// channels).  Non-temporal loads read faster still (6.4 TB/s) but leave X
// out of the last-level cache, and the low-rank product that reads X next
// then took 104 instead of 66 us: the loads stay plain.
template <int PM>
__global__ __launch_bounds__(256) void k_stats_partial(StatsSplitArgs a) {
  __shared__ double red[4][512];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int split = blockIdx.y * 4 + w;
  const int r = blockIdx.z;
  const int64_t c0 = (int64_t)blockIdx.x * 512 + l * 8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (split < a.nsplit && c0 < a.d) {
    const bf16_t* X = a.X + (int64_t)r * a.T * a.d;
    const int64_t t0 = (int64_t)split * a.tchunk;
    const int64_t t1 = min(a.T, t0 + a.tchunk);
    int64_t t = t0;
    for (; t + 4 <= t1; t += 4) {
      u32x4 v0 = *(const u32x4*)(X + (t + 0) * a.d + c0);
      u32x4 v1 = *(const u32x4*)(X + (t + 1) * a.d + c0);
      u32x4 v2 = *(const u32x4*)(X + (t + 2) * a.d + c0);
      u32x4 v3 = *(const u32x4*)(X + (t + 3) * a.d + c0);
      accum8(acc, v0, PM, a.p);
      accum8(acc, v1, PM, a.p);
      accum8(acc, v2, PM, a.p);
      accum8(acc, v3, PM, a.p);
    }
    for (; t < t1; ++t) {
      u32x4 v = *(const u32x4*)(X + t * a.d + c0);
      accum8(acc, v, PM, a.p);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[w][l * 8 + j] = acc[j];
  __syncthreads();
  const int64_t nb = (a.nsplit + 3) / 4;
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int64_t c = (int64_t)blockIdx.x * 512 + i;
    if (c < a.d) {
      const double v = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
      a.partial[((int64_t)r * nb + blockIdx.y) * a.d + c] = v;
    }
  }
}

// One thread per channel; the block partials are read 8 at a time (independent
// loads in flight) and added in slice order.
__global__ __launch_bounds__(64) void k_stats_final(StatsSplitArgs a) {
  const int r = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (c >= a.d) return;
  const int nb = (a.nsplit + 3) / 4;
  const double* P = a.partial + (int64_t)r * nb * a.d + c;
  double S = 0.0;
  int k = 0;
  for (; k + 8 <= nb; k += 8) {
    double v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = P[(int64_t)(k + j) * a.d];
#pragma unroll
    for (int j = 0; j < 8; ++j) S += v[j];
  }
  for (; k < nb; ++k) S += P[(int64_t)k * a.d];
  float dh, dhi;
  diag_half(finish_norm(S, a.pmode, a.p), a.lam, a.alpha, dh, dhi);
  a.dh[(int64_t)r * a.d + c] = dh;
  a.dhi[(int64_t)r * a.d + c] = dhi;
  if (a.dh_export) a.dh_export[(int64_t)r * a.d + c] = dh;
}

hipError_t launch_stats_partial(const StatsSplitArgs& a, int R,
                                const Launch& L) {
  if (a.nsplit == 0) return hipSuccess;
  dim3 grid((unsigned)((a.d + 511) / 512), (unsigned)((a.nsplit + 3) / 4),
            (unsigned)R);
  if (a.pmode == 2) return ext_launch(k_stats_partial<2>, grid, dim3(256), 0, L, a);
  if (a.pmode == 1) return ext_launch(k_stats_partial<1>, grid, dim3(256), 0, L, a);
  return ext_launch(k_stats_partial<0>, grid, dim3(256), 0, L, a);
}

hipError_t launch_stats_final(const StatsSplitArgs& a, int R, const Launch& L) {
  dim3 grid((unsigned)((a.d + 63) / 64), (unsigned)R);
  return ext_launch(k_stats_final, grid, dim3(64), 0, L, a);
}

}  // namespace ttq
