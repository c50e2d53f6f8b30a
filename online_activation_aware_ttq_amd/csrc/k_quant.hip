// Quantize pass of the two-phase (large T) TTQ path on gfx950.
//
// Reads W once and writes the dequantized operand
//   W_hat = (m + s q) D^{-1/2}     rounded once to bf16
// ("TTQ: Activation-Aware Test-Time Quantization ...", gist.science zh
// summary, Sec. 2.1), which the MFMA GEMM then contracts with the raw bf16
// activations.  The codes are decided by the same float32 sequence as the
// fused path (for R requests at once, each with its own statistics and its
// own W_hat).  For quantize-once use it writes the packed codes instead of
// W_hat.  A wave covers 512 consecutive channels of 8 weight rows: each lane
// loads 16 bytes per row, a group of g channels lives in g/8 adjacent
// lanes and is reduced with xor-shuffles inside that lane group.
#include "ttq_internal.h"

namespace ttq {

constexpr int QROWS = 8;  // weight rows per wave (D^{+-1/2} reused across them)

namespace {

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                      false));
}

// min and max over the LPG consecutive lanes of a group: DPP inside each row
// of 16 lanes (quad xor 1 and 2, then the mirrors of 8 and of 16 lanes, each
// of which pairs a lane with one in the other half), a shuffle across rows
template <int LPG>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
  mn = fminf(mn, dpp<0xB1>(mn));   // quad_perm [1,0,3,2]
  mx = fmaxf(mx, dpp<0xB1>(mx));
  if constexpr (LPG >= 4) {
    mn = fminf(mn, dpp<0x4E>(mn));   // quad_perm [2,3,0,1]
    mx = fmaxf(mx, dpp<0x4E>(mx));
  }
  if constexpr (LPG >= 8) {
    mn = fminf(mn, dpp<0x141>(mn));  // row_half_mirror
    mx = fmaxf(mx, dpp<0x141>(mx));
  }
  if constexpr (LPG >= 16) {
    mn = fminf(mn, dpp<0x140>(mn));  // row_mirror
    mx = fmaxf(mx, dpp<0x140>(mx));
  }
  if constexpr (LPG >= 32) {
    mn = fminf(mn, __shfl_xor(mn, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
  }
}

}  // namespace

// CB = 0: write W_hat (and optional byte codes, scales, group offsets; with
// a null W_hat only those exports);
// CB = 1, 2, 4, 8: write the codes packed in CB-bit containers instead of
// W_hat (channel j of a row at bit (j*CB) % 8 of byte (j*CB) / 8).
// QF: the quantizer format (QFmt; W_hat = bf16((c + s L) D^{-1/2})).
// EXP (CB = 0): codes, scales and offsets are asked for; without them the
// integer codes are not formed.
template <int GS, int CB, int QF, bool EXP>
__global__ __launch_bounds__(256) void k_quant(QuantArgs a) {
  constexpr int LPG = GS / 8;
  // W_hat leaves through LDS: lane l quantizes channels 8l .. 8l+7 of the
  // wave's 8 rows, and each store instruction then writes one 64-channel
  // tile slice of all 8 rows (1 KiB contiguous in the tiled layout) rather
  // than 8 pieces of 128 bytes 32 KiB apart
  __shared__ u32x4 tw[4][QROWS][64];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t nchunk = (a.d + 511) / 512;
  const int64_t nblk1 = (((a.d_out + QROWS - 1) / QROWS) * nchunk + 3) / 4;
  // requests one after the other, the last one first: the GEMM that follows
  // starts with request 0, whose W_hat is then the most recently written
  // (still in the last-level cache); W itself is small enough to stay there
  // between the requests
  const int64_t b = blockIdx.x;
  const int xcd = (int)(b & 7);
  const int64_t jb = b >> 3;
  const int64_t nq = (nblk1 + 7) / 8;
  const int64_t bq = (jb % nq) * 8 + xcd;
  const int r = a.R - 1 - (int)(jb / nq);
  if (bq >= nblk1) return;
  const int64_t wid = bq * 4 + w;
  const int64_t rgrp = wid / nchunk;
  const int64_t chunk = wid % nchunk;
  const int64_t row0 = rgrp * QROWS;
  if (row0 >= a.d_out) return;  // uniform over the wave
  const int64_t c0 = chunk * 512 + l * 8;
  const bool live = c0 < a.d;
  const float Nf = a.Nf;
  const float* dhr = a.dh + (int64_t)r * a.d;
  const float* dhir = a.dhi + (int64_t)r * a.d;
  // What == null: the codes, scales and offsets only (no W_hat is written)
  bf16_t* What = a.What ? a.What + (int64_t)r * what_tiled_elems(a.d_out, a.d) : nullptr;
  const int64_t nkw = (a.d + kWtCols - 1) / kWtCols;
  uint8_t* codes_out = a.codes_out ? a.codes_out + (int64_t)r * a.d_out * a.d : nullptr;
  float* s_out = a.s_out ? a.s_out + (int64_t)r * a.d_out * a.G : nullptr;
  float* m_out = a.m_out ? a.m_out + (int64_t)r * a.d_out * a.G : nullptr;

  float dh[8], dhi[8];
  if (live) {
    const f32x4 h0 = *(const f32x4*)(dhr + c0);
    const f32x4 h1 = *(const f32x4*)(dhr + c0 + 4);
    const f32x4 i0 = *(const f32x4*)(dhir + c0);
    const f32x4 i1 = *(const f32x4*)(dhir + c0 + 4);
    dh[0] = h0.x; dh[1] = h0.y; dh[2] = h0.z; dh[3] = h0.w;
    dh[4] = h1.x; dh[5] = h1.y; dh[6] = h1.z; dh[7] = h1.w;
    dhi[0] = i0.x; dhi[1] = i0.y; dhi[2] = i0.z; dhi[3] = i0.w;
    dhi[4] = i1.x; dhi[5] = i1.y; dhi[6] = i1.z; dhi[7] = i1.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) { dh[j] = 0.f; dhi[j] = 0.f; }
  }

  u32x4 wv[QROWS];
#pragma unroll
  for (int rr = 0; rr < QROWS; ++rr) {
    const int64_t row = row0 + rr;
    wv[rr] = (live && row < a.d_out) ? *(const u32x4*)(a.W + row * a.d + c0)
                                     : u32x4{0u, 0u, 0u, 0u};
  }

#pragma unroll
  for (int rr = 0; rr < QROWS; ++rr) {
    const int64_t row = row0 + rr;
    float u[8] = {bf16lo(wv[rr].x) * dh[0], bf16hi(wv[rr].x) * dh[1],
                  bf16lo(wv[rr].y) * dh[2], bf16hi(wv[rr].y) * dh[3],
                  bf16lo(wv[rr].z) * dh[4], bf16hi(wv[rr].z) * dh[5],
                  bf16lo(wv[rr].w) * dh[6], bf16hi(wv[rr].w) * dh[7]};
    float mn = u[0], mx = u[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      mn = fminf(mn, u[j]);
      mx = fmaxf(mx, u[j]);
    }
    group_minmax<LPG>(mn, mx);
    const QGroup gq = qgroup<QF>(mn, mx, Nf);
    const float s = gq.s;
    float q[8];
    unsigned qc[8];
    qlevels8<QF>(gq, u, q);
    if constexpr (CB > 0 || EXP) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qc[j] = qcode<QF>(gq, q[j]);
    }
    if (!live || row >= a.d_out) continue;
    if (CB > 0) {
      // 8 codes of this lane -> 8*CB bits, one aligned store
      uint8_t* dst = a.packed + (int64_t)r * a.d_out * a.row_bytes +
                     row * a.row_bytes + c0 * CB / 8;
      if (CB == 8) {
        u32x2 c;
        c.x = qc[0] | (qc[1] << 8) | (qc[2] << 16) | (qc[3] << 24);
        c.y = qc[4] | (qc[5] << 8) | (qc[6] << 16) | (qc[7] << 24);
        *(u32x2*)dst = c;
      } else {
        unsigned c = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) c |= qc[j] << (j * CB);
        if (CB == 4) *(unsigned*)dst = c;
        else if (CB == 2) *(uint16_t*)dst = (uint16_t)c;
        else *dst = (uint8_t)c;
      }
      if (s_out && (l % LPG) == 0) {
        const int64_t o2 = row * a.G + c0 / GS;
        s_out[o2] = s;
        m_out[o2] = gq.off;
      }
      continue;
    }
    const float c = gq.c;
    u32x4 o;
    o.x = pack_bf16(fmaf(s, q[0], c) * dhi[0], fmaf(s, q[1], c) * dhi[1]);
    o.y = pack_bf16(fmaf(s, q[2], c) * dhi[2], fmaf(s, q[3], c) * dhi[3]);
    o.z = pack_bf16(fmaf(s, q[4], c) * dhi[4], fmaf(s, q[5], c) * dhi[5]);
    o.w = pack_bf16(fmaf(s, q[6], c) * dhi[6], fmaf(s, q[7], c) * dhi[7]);
    if (What) tw[w][rr][l] = o;
    if constexpr (EXP) {
      if (codes_out) {
        u32x2 cc;
        cc.x = qc[0] | (qc[1] << 8) | (qc[2] << 16) | (qc[3] << 24);
        cc.y = qc[4] | (qc[5] << 8) | (qc[6] << 16) | (qc[7] << 24);
        *(u32x2*)(codes_out + row * a.d + c0) = cc;
      }
      if (s_out && (l % LPG) == 0) {
        const int64_t o2 = row * a.G + c0 / GS;
        s_out[o2] = s;
        m_out[o2] = gq.off;
      }
    }
  }
  if (What) {
    const int rr = l >> 3, oc = l & 7;
    const int64_t row = row0 + rr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t c = chunk * 512 + i * 64 + oc * 8;
      if (row < a.d_out && c < a.d)
        *(u32x4*)(What + what_tiled_index(row, c, nkw)) = tw[w][rr][i * 8 + oc];
    }
  }
}

hipError_t launch_quant(const QuantArgs& a, int group, const Launch& L) {
  const int64_t nchunk = (a.d + 511) / 512;
  const int64_t waves = ((a.d_out + QROWS - 1) / QROWS) * nchunk;
  const int64_t nblk1 = (waves + 3) / 4;
  if (nblk1 == 0 || a.R == 0) return hipSuccess;
  const dim3 grid((unsigned)(((nblk1 + 7) / 8) * 8 * a.R)), blk(256);
  const bool exp = a.codes_out != nullptr || a.s_out != nullptr;
#define TTQ_QUANT_CB(GSV, QF)                                                  \
  switch (a.packed ? a.cb : 0) {                                               \
    case 0:                                                                    \
      return exp ? ext_launch(k_quant<GSV, 0, QF, true>, grid, blk, 0, L, a)   \
                 : ext_launch(k_quant<GSV, 0, QF, false>, grid, blk, 0, L, a); \
    case 1: return ext_launch(k_quant<GSV, 1, QF, true>, grid, blk, 0, L, a);  \
    case 2: return ext_launch(k_quant<GSV, 2, QF, true>, grid, blk, 0, L, a);  \
    case 4: return ext_launch(k_quant<GSV, 4, QF, true>, grid, blk, 0, L, a);  \
    case 8: return ext_launch(k_quant<GSV, 8, QF, true>, grid, blk, 0, L, a);  \
    default: return hipErrorInvalidValue;                                      \
  }
#define TTQ_QUANT_GS(GSV)                                                      \
  case GSV:                                                                    \
    switch (a.qf) {                                                            \
      case QF_ASYM: TTQ_QUANT_CB(GSV, QF_ASYM)                                 \
      case QF_SYM: TTQ_QUANT_CB(GSV, QF_SYM)                                   \
      case QF_INTZP: TTQ_QUANT_CB(GSV, QF_INTZP)                               \
      case QF_FP8: TTQ_QUANT_CB(GSV, QF_FP8)                                   \
      default: return hipErrorInvalidValue;                                    \
    }
  switch (group) {
    TTQ_QUANT_GS(32)
    TTQ_QUANT_GS(64)
    TTQ_QUANT_GS(128)
    TTQ_QUANT_GS(256)
    default: return hipErrorInvalidValue;
  }
#undef TTQ_QUANT_GS
#undef TTQ_QUANT_CB
}

}  // namespace ttq
