// Fused single-pass TTQ projection for small token counts (T <= 128).
//
// Each bf16 weight element is read from HBM exactly once.  In registers it
// is scaled by D^{1/2}, the group min/max are reduced, the b-bit code is
// decided in float32 and the contraction with the activations runs on the
// gfx950 matrix cores:
//
//   Y[t,i] = sum_k  s_ik * sum_{j in k} q_ij x'_tj  +  m_ik * sum_{j in k} x'_tj
//
// where x' = x D^{-1/2} and (s_ik, m_ik) are the group scale and minimum
// (for the formats without a real minimum q is the signed level, exact in
// bf16 like the codes, and the m term is absent).
// This is the dequantized product (m + s q) D^{-1/2} X of "TTQ:
// Activation-Aware Test-Time Quantization ..." (gist.science zh summary,
// Sec. 2.1) regrouped so that the integer codes -- exact in bf16 -- are the
// MFMA operand and the per-group affine terms are applied once per group to
// the fp32 accumulators.  The static low-rank term B (A X) (same page, Sec.
// 2.2) is one more MFMA chain on Z = A X.
//
// Activation operand: for T <= 16 one outlier channel can dominate every
// output of a token, so a single bf16 rounding of its x' would be shared by
// all of them; there x' is carried in fp16 (11 significant bits) scaled by a
// power of two per (group, token) so that any float32 magnitude fits, the
// codes are the fp16 operand of v_mfma_f32_16x16x32_f16, and the scale is
// undone in the group epilogue.  (A bf16 pair hi + lo, two MFMAs and twice
// the activation bytes, was 20 % slower on the 8-request 7B-class layer at
// 16 tokens.)  For T > 16 x' is rounded once to bf16 and the rounding errors
// average over the tokens.  It is stored in MFMA
// fragment order so that every activation load is a contiguous 1 KiB per
// wave.  The weights are read with the default cache policy: non-temporal
// loads (meant to keep x', re-read by every workgroup, in L2) made the
// 8-request 7B-class layer 5-8 % slower at 32 and 128 tokens.
//
// MFMA: v_mfma_f32_16x16x32_bf16 with A = x' (16 tokens x 32 channels) and
// B = codes (32 channels x 16 weight rows).  Lane l holds weight row l & 15
// and channels 8*(l >> 4) .. +8 of each 32-channel step -- exactly one 16-byte
// load of W -- so the group statistics of a row live in the 4 lanes
// {l, l^16, l^32, l^48}, and the accumulators of row l & 15 land in the same
// lane that owns its scale and minimum.
//
// Work split: a workgroup of 8 waves owns 16 weight rows (or two blocks of
// 16 that share every activation load, for T > 16 when that still leaves a
// workgroup per CU) and all of K; waves stride over the groups and meet once
// in LDS at the end (fixed order, no inter-workgroup traffic,
// deterministic).  D^{1/2} of the request is staged in LDS once per
// workgroup (when it fits).  Workgroup indices are laid out so that the R
// requests of one weight tile run back to back on the same XCD and share the
// tile through its L2.
#include "ttq_internal.h"

namespace ttq {

constexpr int FW = 8;  // waves per workgroup

// RB: 16-row blocks per workgroup; they share every activation load, which
// divides the activations' L2 -> CU traffic (the binding resource when every
// workgroup re-reads x') by RB.
template <int NTB, int GS, bool DH_LDS, bool EXPORT, int QF, int RB>
__global__ __launch_bounds__(FW * 64) void k_fused(FusedArgs a) {
  constexpr int NKS = GS / 32;
  constexpr bool XF16 = (NTB == 1);  // T <= 16: x' in scaled fp16
  extern __shared__ __attribute__((aligned(16))) float lds[];

  const int64_t b = blockIdx.x;
  const int xcd = (int)(b & 7);
  const int64_t jb = b >> 3;
  const int req = (int)(jb % a.R);
  const int64_t rb0 = ((jb / a.R) * 8 + xcd) * RB;
  if (rb0 >= a.rowblocks) return;

  const int tid = threadIdx.x, l = tid & 63;
  // wave index as a scalar: the group loop below is then wave-uniform control
  // flow (a per-lane counter would make every loop exit a divergent branch)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = l & 15, qd = l >> 4;
  const int64_t T = a.T, d = a.d;
  const int G = a.G;
  const int Tp = NTB * 16;

  const float* dhg = a.dh + (int64_t)req * d;
  const bf16_t* xs = a.xs + (int64_t)req * Tp * d;
  const float* sx = a.sx + (int64_t)req * G * Tp;
  const float* xsc = XF16 ? a.xsc + (int64_t)req * G * Tp : nullptr;
  // each row block's weight rows as one bounded buffer: rows past d_out and
  // groups past the end read as zeros without memory traffic (separate
  // scalars rather than an array or structure: see the persistent GEMM)
  const int64_t rh0 = min((int64_t)16, a.d_out - rb0 * 16);
  const int64_t rh1 = RB > 1 ? max((int64_t)0, min((int64_t)16, a.d_out - (rb0 + 1) * 16)) : 0;
  const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(a.W + rb0 * 16 * d, (uint32_t)(rh0 * d * 2));
  const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(a.W + (rb0 + (RB > 1 ? 1 : 0)) * 16 * d,
                                               (uint32_t)(rh1 * d * 2));
  const uint32_t lane_off = (uint32_t)((lr * d + qd * 8) * 2);
  const float Nf = a.Nf;

  f32x4 acc[RB][NTB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[r][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // T <= 16: lane l holds token l & 15 of the activation operand (scaled
  // fp16), and the inverse scales of tokens 4 (l >> 4) .. +4
  u32x4 xh[NKS];
  f32x4 sxv0, scv0;

  auto load_w = [&](u32x4 (&wv)[RB][NKS], int g) {
    const uint32_t soff = g < G ? (uint32_t)g * GS * 2 : kOutOfRange;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int k = 0; k < NKS; ++k)
        wv[r][k] = buf_load16(r ? wr1 : wr0, lane_off + k * 64, soff);
  };
  // fragment-ordered x' (zero past T): each load is 1 KiB per wave
  auto load_x = [&](int g) {
    if (NTB == 1) {
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        const int64_t fi = 8 * xs_frag_index(g, 0, k, l, 1, GS);
        xh[k] = *(const u32x4*)(xs + fi);
      }
      sxv0 = *(const f32x4*)(sx + (int64_t)g * Tp + qd * 4);
      scv0 = *(const f32x4*)(xsc + (int64_t)g * Tp + qd * 4);
    }
  };

  auto process = [&](const u32x4 (&wv)[RB][NKS], int g) {
    const int64_t colg = (int64_t)g * GS + qd * 8;
    u32x4 qv[RB][NKS];
    float sr[RB], mcr[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t row = (rb0 + r) * 16 + lr;
      const bool row_ok = row < a.d_out;
      // u = fl(w * dh), group min / max
      float u[NKS][8];
      float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        f32x4 d0, d1;
        if (DH_LDS) {
          d0 = *(const f32x4*)(lds + colg + k * 32);
          d1 = *(const f32x4*)(lds + colg + k * 32 + 4);
        } else {
          d0 = *(const f32x4*)(dhg + colg + k * 32);
          d1 = *(const f32x4*)(dhg + colg + k * 32 + 4);
        }
        u[k][0] = bf16lo(wv[r][k].x) * d0.x;
        u[k][1] = bf16hi(wv[r][k].x) * d0.y;
        u[k][2] = bf16lo(wv[r][k].y) * d0.z;
        u[k][3] = bf16hi(wv[r][k].y) * d0.w;
        u[k][4] = bf16lo(wv[r][k].z) * d1.x;
        u[k][5] = bf16hi(wv[r][k].z) * d1.y;
        u[k][6] = bf16lo(wv[r][k].w) * d1.z;
        u[k][7] = bf16hi(wv[r][k].w) * d1.w;
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

      // s = fl(fl(M - m) / N), inv = fl(1 / s); IEEE division, no
      // contraction (other formats: see QFmt)
      const QGroup gq = qgroup<QF>(mn, mx, Nf);
      const float inv = gq.inv;
      sr[r] = gq.s;

      // codes q = rint(fl(fl(u - m) * inv)), packed as bf16 pairs.  The clamp
      // to [0, N] of the definition is a no-op here: 0 <= u - m <= M - m, and
      // the largest t is N (1 + e) with |e| < 4e-7 for the three roundings,
      // so rint(t) stays in [0, N] for every finite input (NaN propagates to
      // Y).
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        float q[8];
        if constexpr (QF == QF_ASYM) {
#pragma unroll
          for (int j = 0; j < 8; ++j) q[j] = __builtin_rintf((u[k][j] - mn) * inv);
        } else {
          qlevels8<QF>(gq, u[k], q);
        }
        if constexpr (XF16) {
          // fp16 operand (levels and E4M3 values are exact in fp16)
          qv[r][k].x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(q[0], q[1]));
          qv[r][k].y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(q[2], q[3]));
          qv[r][k].z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(q[4], q[5]));
          qv[r][k].w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(q[6], q[7]));
        } else {
          qv[r][k].x = __builtin_amdgcn_perm(__float_as_uint(q[1]),
                                             __float_as_uint(q[0]), 0x07060302u);
          qv[r][k].y = __builtin_amdgcn_perm(__float_as_uint(q[3]),
                                             __float_as_uint(q[2]), 0x07060302u);
          qv[r][k].z = __builtin_amdgcn_perm(__float_as_uint(q[5]),
                                             __float_as_uint(q[4]), 0x07060302u);
          qv[r][k].w = __builtin_amdgcn_perm(__float_as_uint(q[7]),
                                             __float_as_uint(q[6]), 0x07060302u);
        }
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
        const int64_t o = ((int64_t)req * a.d_out + row) * G + g;
        a.s_out[o] = gq.s;
        a.m_out[o] = gq.off;
      }
      mcr[r] = QF == QF_ASYM ? mn : 0.f;
    }

    // contraction on the matrix cores + per-group affine epilogue
    if (NTB == 1) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < NKS; ++k)
          P = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(f16x8, xh[k]), __builtin_bit_cast(f16x8, qv[r][k]), P,
              0, 0, 0);
        // undo the token's power-of-two scale (exact), then s P + m sum(x')
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[r][0][i] = fmaf(sr[r], P[i] * scv0[i], fmaf(mcr[r], sxv0[i], acc[r][0][i]));
      }
    } else {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        // fragment-ordered x' (zero past T): each load is 1 KiB per wave,
        // shared by the RB row blocks
        u32x4 xv[NKS];
#pragma unroll
        for (int k = 0; k < NKS; ++k)
          xv[k] = *(const u32x4*)(xs + 8 * xs_frag_index(g, tb, k, l, NTB, GS));
        const f32x4 sxv = *(const f32x4*)(sx + (int64_t)g * Tp + tb * 16 + qd * 4);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k = 0; k < NKS; ++k)
            P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, xv[k]),
                __builtin_bit_cast(bf16x8, qv[r][k]), P, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[r][tb][i] = fmaf(sr[r], P[i], fmaf(mcr[r], sxv[i], acc[r][tb][i]));
        }
      }
    }
  };

  // two weight register sets in ping-pong: the loads of the next group are
  // issued after this group's activation loads, so waiting for the latter
  // does not wait for the former, and no register copies are needed
  // (a prefetch past the last group is out of range: zeros, no traffic)
  // static low-rank term B (A X): one more MFMA chain on Z = A X, rank step
  // kk (32 columns) per wave.  Bounded buffer loads: rows past d_out,
  // columns past the rank and tokens past T read zeros with no branch.
  constexpr uint32_t kPastEnd = 0xFFFFFFF0u;
  const int nk = a.rank > 0 ? a.rp / 32 : 0;
  const int64_t lr_rows = min((int64_t)16 * RB, a.d_out - rb0 * 16);
  const __amdgpu_buffer_rsrc_t brs =
      make_rsrc(a.rank > 0 ? a.Blr + rb0 * 16 * a.rank : a.W,
                a.rank > 0 ? (uint32_t)(lr_rows * a.rank * 2) : 0u);
  const __amdgpu_buffer_rsrc_t zrs =
      make_rsrc(a.rank > 0 ? a.Z + (int64_t)req * T * a.rp : a.W,
                a.rank > 0 ? (uint32_t)(T * a.rp * 2) : 0u);
  auto lr_load = [&](int kk, u32x4 (&bv)[RB], u32x4 (&zv)[NTB]) {
    const int c8 = kk * 32 + qd * 8;
    const bool on = kk < nk && c8 < a.rank;
#pragma unroll
    for (int r = 0; r < RB; ++r)
      bv[r] = buf_load16(brs, on ? (uint32_t)(((r * 16 + lr) * a.rank + c8) * 2) : kPastEnd, 0);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
      zv[tb] = buf_load16(zrs, kk < nk ? (uint32_t)(((tb * 16 + lr) * a.rp + c8) * 2) : kPastEnd, 0);
  };
  auto lr_mfma = [&](const u32x4 (&bv)[RB], const u32x4 (&zv)[NTB]) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int r = 0; r < RB; ++r)
        acc[r][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, zv[tb]), __builtin_bit_cast(bf16x8, bv[r]),
            acc[r][tb], 0, 0, 0);
  };
  u32x4 lbv[RB], lzv[NTB];

  u32x4 wa[RB][NKS], wb[RB][NKS];
  int g = w;
  if (DH_LDS) {
    // D^{1/2} of this request into LDS before the first weight loads: once
    // every CU's weight requests are queued, these small reads would sit
    // behind them
    for (int64_t c = (int64_t)tid * 4; c < d; c += FW * 64 * 4)
      *(f32x4*)(lds + c) = *(const f32x4*)(dhg + c);
    wait_vmem_all();
    __builtin_amdgcn_sched_barrier(0);
    load_w(wa, g);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  } else {
    load_w(wa, g);
  }
  // (scheduling barriers keep that issue order: the compiler would otherwise
  // hoist loads across the prefetch)
  while (g < G) {
    load_x(g);
    __builtin_amdgcn_sched_barrier(0);
    load_w(wb, g + FW);
    __builtin_amdgcn_sched_barrier(0);
    process(wa, g);
    g += FW;
    if (g >= G) break;
    load_x(g);
    __builtin_amdgcn_sched_barrier(0);
    load_w(wa, g + FW);
    __builtin_amdgcn_sched_barrier(0);
    process(wb, g);
    g += FW;
  }

  // the low-rank steps of this wave, in increasing kk (requesting the first
  // step's operands with the first weights instead raised the register count
  // at T <= 16 from 123 to 131 and cost a workgroup per CU: +29 % at 8 x 16
  // tokens)
  for (int kk = w; kk < nk; kk += FW) {
    lr_load(kk, lbv, lzv);
    lr_mfma(lbv, lzv);
  }

  // combine the 8 waves in a fixed order, one row block at a time (LDS reused
  // after the main loop)
  float* Y = a.Y + (int64_t)req * T * a.d_out;
  float* red = lds;  // [FW][NTB * 4][64]
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if (DH_LDS || r > 0) __syncthreads();
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(w * NTB * 4 + tb * 4 + i) * 64 + l] = acc[r][tb][i];
    __syncthreads();
    for (int e = tid; e < NTB * 256; e += FW * 64) {
      const int ti = e >> 6, ll = e & 63;
      const int64_t tok = (ti >> 2) * 16 + (ll >> 4) * 4 + (ti & 3);
      const int64_t rowx = (rb0 + r) * 16 + (ll & 15);
      if (tok < T && rowx < a.d_out) {
        float v = red[ti * 64 + ll];
#pragma unroll
        for (int ww = 1; ww < FW; ++ww) v += red[(ww * NTB * 4 + ti) * 64 + ll];
        Y[tok * a.d_out + rowx] = v;
      }
    }
  }
}

template <int NTB, bool DHL, int QF, int RB>
static hipError_t launch_fused_ntb(const FusedArgs& a, int group, dim3 grid,
                                   uint32_t lds, const Launch& L) {
  const dim3 blk(FW * 64);
  // the exports are a separate instantiation: conditional stores in the loop
  // would make the compiler's memory wait counts conservative
  const bool exp = a.codes_out || a.s_out;
#define TTQ_FUSED_CASE(GSV)                                                    \
  case GSV:                                                                    \
    return exp ? ext_launch(k_fused<NTB, GSV, DHL, true, QF, RB>, grid, blk,   \
                            lds, L, a)                                         \
               : ext_launch(k_fused<NTB, GSV, DHL, false, QF, RB>, grid, blk,  \
                            lds, L, a);
  switch (group) {
    TTQ_FUSED_CASE(32)
    TTQ_FUSED_CASE(64)
    TTQ_FUSED_CASE(128)
    case 256:
      // two row blocks of 256-channel groups would not fit in registers
      if constexpr (RB == 1) {
        return exp ? ext_launch(k_fused<NTB, 256, DHL, true, QF, 1>, grid, blk,
                                lds, L, a)
                   : ext_launch(k_fused<NTB, 256, DHL, false, QF, 1>, grid, blk,
                                lds, L, a);
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
#undef TTQ_FUSED_CASE
}

template <bool DHL, int QF, int RB>
static hipError_t launch_fused_rb(const FusedArgs& a, int ntb, int group,
                                  dim3 grid, uint32_t lds, const Launch& L) {
  switch (ntb) {
    case 1:
      // (one token tile: the kernel is bound by its vector ALU work, and the
      // host takes one row block)
      if constexpr (RB == 1) return launch_fused_ntb<1, DHL, QF, 1>(a, group, grid, lds, L);
      return hipErrorInvalidValue;
    case 2: return launch_fused_ntb<2, DHL, QF, RB>(a, group, grid, lds, L);
    case 4: return launch_fused_ntb<4, DHL, QF, RB>(a, group, grid, lds, L);
    case 8: return launch_fused_ntb<8, DHL, QF, RB>(a, group, grid, lds, L);
    default: return hipErrorInvalidValue;
  }
}

template <bool DHL, int QF>
static hipError_t launch_fused_qf(const FusedArgs& a, int ntb, int group, int rb,
                                  dim3 grid, uint32_t lds, const Launch& L) {
  return rb == 2 ? launch_fused_rb<DHL, QF, 2>(a, ntb, group, grid, lds, L)
                 : launch_fused_rb<DHL, QF, 1>(a, ntb, group, grid, lds, L);
}

template <bool DHL>
static hipError_t launch_fused_dhl(const FusedArgs& a, int ntb, int group, int rb,
                                   dim3 grid, uint32_t lds, const Launch& L) {
  switch (a.qf) {
    case QF_ASYM: return launch_fused_qf<DHL, QF_ASYM>(a, ntb, group, rb, grid, lds, L);
    case QF_SYM: return launch_fused_qf<DHL, QF_SYM>(a, ntb, group, rb, grid, lds, L);
    case QF_INTZP: return launch_fused_qf<DHL, QF_INTZP>(a, ntb, group, rb, grid, lds, L);
    case QF_FP8: return launch_fused_qf<DHL, QF_FP8>(a, ntb, group, rb, grid, lds, L);
    default: return hipErrorInvalidValue;
  }
}

size_t fused_lds_bytes(int64_t d, int ntb, bool* dh_in_lds) {
  const size_t red = (size_t)FW * ntb * 4 * 64 * sizeof(float);
  const size_t dhb = (size_t)d * sizeof(float);
  *dh_in_lds = dhb <= kFusedDhLdsMax;
  return *dh_in_lds ? (dhb > red ? dhb : red) : red;
}

hipError_t launch_fused(const FusedArgs& a, int ntb, int group, int rb,
                        const Launch& L) {
  if (rb != 1 && rb != 2) return hipErrorInvalidValue;
  const int64_t pairs = (a.rowblocks + rb - 1) / rb;
  const int64_t nblk = ((pairs + 7) / 8) * 8 * a.R;
  if (nblk == 0) return hipSuccess;
  bool dh_in = false;
  const uint32_t lds = (uint32_t)fused_lds_bytes(a.d, ntb, &dh_in);
  dim3 grid((unsigned)nblk);
  return dh_in ? launch_fused_dhl<true>(a, ntb, group, rb, grid, lds, L)
               : launch_fused_dhl<false>(a, ntb, group, rb, grid, lds, L);
}

}  // namespace ttq
