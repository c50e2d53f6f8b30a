// Single-launch TTQ projection for one token (T = 1, decode).
//
// With one token the whole call is one pass over W, so everything runs in
// one kernel: every workgroup derives the statistics of the token itself
// (for T = 1 the channel norm is |x_j| for every p), keeps D^{1/2} and
// x' = x D^{-1/2} in LDS, and streams its 16 weight rows exactly once:
//
//   y_i = sum_k  s_ik * sum_{j in k} q_ij x'_j  +  m_ik * sum_{j in k} x'_j
//
// the dequantized product (m + s q) D^{-1/2} x of "TTQ: Activation-Aware
// Test-Time Quantization ..." (gist.science zh summary, Sec. 2.1), with the
// per-group affine terms applied once per group (for the formats without a
// real minimum, q is the signed level and the m term is absent).  x' stays in float32 and
// the dot products run on the VALU (a 16x16 MFMA tile would be 1/16 used),
// so the activation operand is never rounded to bf16.
//
// D^{1/2} is evaluated exactly as in the statistics kernels (float64 norm
// and power, one rounding to float32), so the codes are decided from the
// same float32 values as on the other paths.
//
// Lane layout: lane l holds weight row l & 15 and channels 8*(l >> 4) .. +8
// of each 32-channel step (one 16-byte load of W);
// a group's statistics live in lanes {l, l^16, l^32, l^48}.  Each of the 16
// waves owns a contiguous run of groups (contiguous weight bytes per row),
// derives the statistics of its own channels while its first weights are in
// flight, and then requests each next group as soon as the current one has
// been processed.  The whole matrix is in flight across the chip either way;
// measured on MI355X, a second group in flight per wave (requested before
// the current one is processed, or before the statistics) makes the call
// slower, not faster.  The statistics and every weight request run at raised
// wave priority, so requests are not held behind other waves' arithmetic.
// Weights are read with bounded buffer loads: a request past the last group
// returns zeros without memory traffic, so the loop needs no branches.
#include "ttq_internal.h"

namespace ttq {


// D^{1/2} for one channel of one token, float64.  For T = 1 the norm is |x|
// for p in {1, 2}; the general route mirrors the reduction kernels.  FAST
// (p in {1, 2} and alpha in {0, 1/2, 1, 2}) uses square roots instead of
// pow: correctly rounded ones for alpha = 1 and, outside [1e-30, 1e30], for
// alpha = 1/2; inside that range base^(1/4) is a float32 seed (two square
// roots) refined by one Newton step in float64, z + z e / 4 with
// e = (base - z^4) / z^4 (e of order 2^-21; the neglected terms, about
// 3 e^2 / 32, stay below 2^-40 relative even with a seed a few ulps off).
// Such a value rounds to the same float32 as the float64 route unless it
// lies within that distance of a rounding midpoint; for every bf16 input
// at the lambdas checked the results are equal.  The kernel's workgroups each derive
// the statistics of their token, so this is their prologue's main cost.
template <bool FAST>
__device__ __forceinline__ double gemv_diag(double ax, int pmode, double p,
                                            double lam, double alpha) {
  double n = ax;
  if (!FAST && pmode == 0 && ax != 0.0) n = pow(pow(ax, p), 1.0 / p);
  const double base = n + lam;
  if (!(base > 0.0) || alpha == 0.0) return 1.0;
  if (!FAST) return pow(base, 0.5 * alpha);
  if (alpha == 0.5) {
    if (base >= 1e-30 && base <= 1e30) {
      const double z = (double)__builtin_amdgcn_sqrtf(__builtin_amdgcn_sqrtf((float)base));
      const double z4 = (z * z) * (z * z);
      const double e = (double)((float)(base - z4) * __builtin_amdgcn_rcpf((float)z4));
      return z + z * (e * 0.25);
    }
    return sqrt(sqrt(base));
  }
  if (alpha == 1.0) return sqrt(base);
  return base;  // alpha == 2
}

// Waves per workgroup: 16 where the registers fit in the 128 VGPRs of a
// 1024-thread workgroup (the timed variants up to g = 128), else 8.
template <int GS, bool EXPORT>
constexpr int gemv_waves() {
  return (GS <= 128 && !EXPORT) ? 16 : 8;
}

template <int GS, bool FAST, bool EXPORT, int QF>
__global__ __launch_bounds__((gemv_waves<GS, EXPORT>() * 64)) void k_gemv(
    GemvArgs a) {
  constexpr int VW = gemv_waves<GS, EXPORT>();
  constexpr int NKS = GS / 32;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  // LDS: dh[d] | xp[d] | sxp[G] | red[VW][16]
  const int64_t d = a.d;
  const int G = a.G;
  float* dh_s = lds;
  float* xp_s = lds + d;
  float* sx_s = lds + 2 * d;
  float* red = sx_s + G;

  const int64_t b = blockIdx.x;
  const int xcd = (int)(b & 7);
  const int64_t jb = b >> 3;
  const int64_t rb = (jb / a.R) * 8 + xcd;
  const int req = (int)(jb % a.R);
  if (rb >= a.rowblocks) return;

  // the statistics prologue and the weight requests go first (see above)
  __builtin_amdgcn_s_setprio(2);
  const int tid = threadIdx.x, l = tid & 63;
  // wave index as a scalar: the group loop below is then wave-uniform control
  // flow (a per-lane counter would make every loop exit a divergent branch)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = l & 15, qd = l >> 4;
  const int64_t row = rb * 16 + lr;
  const bool row_ok = row < a.d_out;
  const bf16_t* x = a.X + (int64_t)req * d;
  const float Nf = a.Nf;

  // the workgroup's weight rows as one bounded buffer: rows past d_out and
  // groups past the end read as zeros without memory traffic
  const int64_t rows_here = min((int64_t)16, a.d_out - rb * 16);
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(a.W + rb * 16 * d, (uint32_t)(rows_here * d * 2));
  const uint32_t lane_off = (uint32_t)((lr * d + qd * 8) * 2);
  auto load_w = [&](u32x4 (&wv)[NKS], int g) {
    const uint32_t soff = g < G ? (uint32_t)g * GS * 2 : kOutOfRange;
#pragma unroll
    for (int k = 0; k < NKS; ++k) wv[k] = buf_load16(wr, lane_off + k * 64, soff);
  };

  // ---- prologue, per wave (no workgroup barrier).  Wave w owns the
  // contiguous groups [w*NGW, (w+1)*NGW) and derives the statistics of
  // exactly those channels:
  //   D^{1/2}  float64, rounded once (it decides the codes)
  //   x' = x D^{-1/2} (float32; it only enters the contraction)
  //   group sums of x'
  // Loads complete in issue order within a wave, so the token's channels are
  // requested first and the weight ring right after: waiting for the token
  // then leaves the weight loads in flight, and the float64 work overlaps
  // them.  Token layout: piece p holds channels p*256 + 4*l .. +4 of the
  // wave's run; a group spans GS / 4 adjacent lanes of one piece.
  const int NGW = (G + VW - 1) / VW;
  const int g_begin = w * NGW;
  const int g_end = min(G, g_begin + NGW);
  constexpr int NP = (int)(kGemvMaxD / (VW * 256));   // token pieces per lane
  static_assert(NP * VW * 256 == kGemvMaxD, "token pieces");
  const int64_t c_begin = (int64_t)g_begin * GS;
  const int64_t c_end = (int64_t)g_end * GS;
  u32x2 xv[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t c = c_begin + p * 256 + l * 4;
    xv[p] = *(const u32x2*)(x + (c < c_end ? c : 0));
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 wv[NKS];
  int g = g_begin;
  load_w(wv, g < g_end ? g : G);
  __builtin_amdgcn_sched_barrier(0);
  // low-rank operands (bounded loads: rows past d_out and columns past the
  // rank read zeros with no branch)
  constexpr uint32_t kPastEnd = 0xFFFFFFF0u;
  const __amdgpu_buffer_rsrc_t brs =
      make_rsrc(a.rank > 0 ? a.Blr + rb * 16 * a.rank : a.W,
                a.rank > 0 ? (uint32_t)(rows_here * a.rank * 2) : 0u);
  const __amdgpu_buffer_rsrc_t zrs =
      make_rsrc(a.rank > 0 ? a.Z + (int64_t)req * a.rp : a.W,
                a.rank > 0 ? (uint32_t)(a.rank * 2) : 0u);
  const int lr_k0 = (w * 4 + qd) * 8;
  auto lr_load = [&](int k, u32x4& bv, u32x4& zv) {
    const bool on = k < a.rank;
    bv = buf_load16(brs, on ? (uint32_t)((lr * a.rank + k) * 2) : kPastEnd, 0);
    zv = buf_load16(zrs, on ? (uint32_t)(k * 2) : kPastEnd, 0);
  };
  auto lr_fma = [](float& acc_, const u32x4& bv, const u32x4& zv) {
    acc_ = fmaf(bf16lo(bv.x), bf16lo(zv.x), acc_);
    acc_ = fmaf(bf16hi(bv.x), bf16hi(zv.x), acc_);
    acc_ = fmaf(bf16lo(bv.y), bf16lo(zv.y), acc_);
    acc_ = fmaf(bf16hi(bv.y), bf16hi(zv.y), acc_);
    acc_ = fmaf(bf16lo(bv.z), bf16lo(zv.z), acc_);
    acc_ = fmaf(bf16hi(bv.z), bf16hi(zv.z), acc_);
    acc_ = fmaf(bf16lo(bv.w), bf16lo(zv.w), acc_);
    acc_ = fmaf(bf16hi(bv.w), bf16hi(zv.w), acc_);
  };
  u32x4 lbv = {0u, 0u, 0u, 0u}, lzv = {0u, 0u, 0u, 0u};
  if (a.rank > 0) lr_load(lr_k0, lbv, lzv);   // (uniform)
  __builtin_amdgcn_sched_barrier(0);
  constexpr int lpg4 = GS / 4;  // lanes per group
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (c_begin + p * 256 >= c_end) break;  // wave-uniform
    const int64_t c = c_begin + p * 256 + l * 4;
    const float xf[4] = {bf16lo(xv[p].x), bf16hi(xv[p].x), bf16lo(xv[p].y),
                         bf16hi(xv[p].y)};
    float hv[4], xpv[4];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hv[j] = (float)gemv_diag<FAST>(fabs((double)xf[j]), a.pmode, a.p, a.lam,
                                     a.alpha);
      xpv[j] = xf[j] * __builtin_amdgcn_rcpf(hv[j]);
      ps += xpv[j];
    }
    if (c < c_end) {
      *(f32x4*)(dh_s + c) = f32x4{hv[0], hv[1], hv[2], hv[3]};
      *(f32x4*)(xp_s + c) = f32x4{xpv[0], xpv[1], xpv[2], xpv[3]};
      if (EXPORT && a.dh_export && rb == 0)
        *(f32x4*)(a.dh_export + (int64_t)req * d + c) =
            f32x4{hv[0], hv[1], hv[2], hv[3]};
    }
#pragma unroll
    for (int off = lpg4 >> 1; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    if (c < c_end && (l % lpg4) == 0) sx_s[c / GS] = ps;
  }
  // the wave reads back only what it wrote: LDS operations of one wave
  // complete in order, so a wave-level fence suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- main loop: quantize-dequantize + dot, one group per step
  float acc = 0.f;
  auto process = [&](const u32x4 (&wv)[NKS], int gg) {
    const int64_t colg = (int64_t)gg * GS + qd * 8;
    float u[NKS][8];
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < NKS; ++k) {
      const f32x4 d0 = *(const f32x4*)(dh_s + colg + k * 32);
      const f32x4 d1 = *(const f32x4*)(dh_s + colg + k * 32 + 4);
      u[k][0] = bf16lo(wv[k].x) * d0.x;
      u[k][1] = bf16hi(wv[k].x) * d0.y;
      u[k][2] = bf16lo(wv[k].y) * d0.z;
      u[k][3] = bf16hi(wv[k].y) * d0.w;
      u[k][4] = bf16lo(wv[k].z) * d1.x;
      u[k][5] = bf16hi(wv[k].z) * d1.y;
      u[k][6] = bf16lo(wv[k].w) * d1.z;
      u[k][7] = bf16hi(wv[k].w) * d1.w;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mn = fminf(mn, u[k][j]);
        mx = fmaxf(mx, u[k][j]);
      }
    }
    mn = fminf(mn, __shfl_xor(mn, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mn = fminf(mn, __shfl_xor(mn, 32));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // s = fl(fl(M - m) / N), inv = fl(1 / s); IEEE division, no contraction
    // (other formats: see QFmt)
    const QGroup gq = qgroup<QF>(mn, mx, Nf);
    const float s = gq.s;
    const float inv = gq.inv;
    // q = rint(fl(fl(u - m) * inv)) (the clamp to [0, N] is a no-op, see the
    // fused kernel); P = sum q x' over this lane's 32 channels
    float P = 0.f;
#pragma unroll
    for (int k = 0; k < NKS; ++k) {
      const f32x4 x0 = *(const f32x4*)(xp_s + colg + k * 32);
      const f32x4 x1 = *(const f32x4*)(xp_s + colg + k * 32 + 4);
      const float xq[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      float q[8];
      if constexpr (QF == QF_ASYM) {
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = __builtin_rintf((u[k][j] - mn) * inv);
      } else {
        qlevels8<QF>(gq, u[k], q);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) P = fmaf(q[j], xq[j], P);
      if (EXPORT && a.codes_out && row_ok) {
        u32x2 c;
        c.x = qcode<QF>(gq, q[0]) | (qcode<QF>(gq, q[1]) << 8) |
              (qcode<QF>(gq, q[2]) << 16) | (qcode<QF>(gq, q[3]) << 24);
        c.y = qcode<QF>(gq, q[4]) | (qcode<QF>(gq, q[5]) << 8) |
              (qcode<QF>(gq, q[6]) << 16) | (qcode<QF>(gq, q[7]) << 24);
        *(u32x2*)(a.codes_out + ((int64_t)req * a.d_out + row) * d + colg +
                  k * 32) = c;
      }
    }
    if (EXPORT && a.s_out && row_ok && qd == 0) {
      const int64_t o = ((int64_t)req * a.d_out + row) * G + gg;
      a.s_out[o] = s;
      a.m_out[o] = gq.off;
    }
    acc = fmaf(s, P, acc);
    if (QF == QF_ASYM && qd == 0) acc = fmaf(mn, sx_s[gg], acc);
  };

  // one group at a time: process it, then request the next one (past the
  // run: an empty request) at raised priority
  __builtin_amdgcn_s_setprio(0);
  while (g < g_end) {
    process(wv, g);
    g += 1;
    __builtin_amdgcn_s_setprio(2);
    load_w(wv, g < g_end ? g : G);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  }

  // static low-rank term: + B[row, :] . z, z = A x precomputed.  Lane
  // quarter qd of wave w takes columns (4w + qd) * 8 + 512 j .. +8, so a
  // rank of up to 512 is one step; the first step's operands were requested
  // with the first weights
  if (a.rank > 0) {
    lr_fma(acc, lbv, lzv);
    for (int k = lr_k0 + VW * 32; k < a.rank; k += VW * 32) {
      u32x4 bv, zv;
      lr_load(k, bv, zv);
      lr_fma(acc, bv, zv);
    }
  }

  // reduce: the 4 lanes of a row (fixed xor order), then the 8 waves
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (qd == 0) red[w * 16 + lr] = acc;
  __syncthreads();
  if (tid < 16) {
    float v = red[tid];
#pragma unroll
    for (int ww = 1; ww < VW; ++ww) v += red[ww * 16 + tid];
    const int64_t rowx = rb * 16 + tid;
    if (rowx < a.d_out) a.Y[(int64_t)req * a.d_out + rowx] = v;
  }
}

size_t gemv_lds_bytes(int64_t d, int G) {
  return (size_t)(2 * d + G + 16 * 16) * sizeof(float);
}

hipError_t launch_gemv(const GemvArgs& a, int group, const Launch& L) {
  const int64_t nblk = ((a.rowblocks + 7) / 8) * 8 * a.R;
  if (nblk == 0) return hipSuccess;
  if (a.d > kGemvMaxD) return hipErrorInvalidValue;
  const uint32_t lds = (uint32_t)gemv_lds_bytes(a.d, a.G);
  const dim3 grid((unsigned)nblk);
  const bool fast = a.pmode != 0 && (a.alpha == 0.0 || a.alpha == 0.5 ||
                                     a.alpha == 1.0 || a.alpha == 2.0);
  // optional exports (codes, scales, minima, D^{1/2}) are a separate
  // instantiation: conditional stores in the loop would make the compiler's
  // memory wait counts conservative on the timed path
  const bool exp = a.codes_out || a.s_out || a.dh_export;
#define TTQ_GEMV_LAUNCH(GSV, F, E, QF)                                        \
  ext_launch(k_gemv<GSV, F, E, QF>, grid, dim3(gemv_waves<GSV, E>() * 64), lds, \
             L, a)
#define TTQ_GEMV_FE(GSV, QF)                                                  \
  if (exp)                                                                    \
    return fast ? TTQ_GEMV_LAUNCH(GSV, true, true, QF)                        \
                : TTQ_GEMV_LAUNCH(GSV, false, true, QF);                      \
  return fast ? TTQ_GEMV_LAUNCH(GSV, true, false, QF)                         \
              : TTQ_GEMV_LAUNCH(GSV, false, false, QF);
#define TTQ_GEMV_CASE(GSV)                                                    \
  case GSV:                                                                   \
    switch (a.qf) {                                                           \
      case QF_ASYM: TTQ_GEMV_FE(GSV, QF_ASYM)                                 \
      case QF_SYM: TTQ_GEMV_FE(GSV, QF_SYM)                                   \
      case QF_INTZP: TTQ_GEMV_FE(GSV, QF_INTZP)                               \
      case QF_FP8: TTQ_GEMV_FE(GSV, QF_FP8)                                   \
      default: return hipErrorInvalidValue;                                   \
    }
  switch (group) {
    TTQ_GEMV_CASE(32)
    TTQ_GEMV_CASE(64)
    TTQ_GEMV_CASE(128)
    TTQ_GEMV_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef TTQ_GEMV_CASE
#undef TTQ_GEMV_FE
#undef TTQ_GEMV_LAUNCH
}

}  // namespace ttq
