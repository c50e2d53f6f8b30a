// Projection GEMM that quantizes its weight tiles itself (gfx950):
//
//   C[M][N] = X[M][K1] * W_hat[N][K1]^T  +  A2[M][K2] * B2[N][K2]^T
//
// with W_hat = (m + s q) D^{-1/2} rounded once to bf16, the dequantized
// weights of "TTQ: Activation-Aware Test-Time Quantization ..." (gist.science
// zh summary, Sec. 2.1): the weight tile is read from HBM as bf16, scaled by
// D^{1/2}, reduced to group minima and maxima, coded and dequantized in
// registers and written to LDS as the MFMA operand.  No W_hat array exists in
// HBM, so for a few token tiles per weight tile this replaces a full pass that
// writes and re-reads the dequantized weights.  The float32 decision sequence
// and the bf16 rounding are those of the quantize pass, so the product equals
// quantize pass + GEMM bit for bit.
//
// Tile: 256 tokens x 128 weight rows, 8 waves (two per SIMD: one wave's
// quantization arithmetic issues while the other's MFMAs run), each wave
// 64 x 64 outputs with v_mfma_f32_32x32x16_bf16.  LDS (160 KB):
//  * three 32 KB stages of the activation tile (64 channels), filled by
//    buffer_load ... lds two k-tiles ahead;
//  * two 32 KB weight chunks of 128 channels (two k-tiles), written by the
//    waves' own quantization: while the matrix cores work on chunk c, the
//    same waves quantize chunk c+1 (64 rows in each of its two k-tiles) with
//    the weights of three k-tiles later in flight.
// Both operands use 128-byte LDS rows with XOR-swizzled 16-byte chunks.
// A quantization job (64 rows x 128 channels) gives each lane one row x 16
// channels: lane p of an 8-lane set holds channels 8p..8p+7 of both k-tile
// halves, so one wave load covers 8 rows x 128 contiguous bytes.  Group
// minima and maxima are reduced across the 8 (or 4) lanes of a group with
// DPP; with two groups per lane, each lane of a quad divides for one and the
// quad broadcasts the results.
// The low-rank segment (K2, already bf16) follows the main loop, copied into
// the weight chunks by buffer_load ... lds.
#include <type_traits>

#include "ttq_internal.h"

namespace ttq {

namespace {

constexpr int QBM = 256, QBN = 128, QBK = 64;
constexpr int QNS = 3;                       // activation stages
constexpr int QNW = 8;                       // waves
constexpr int QA_BYTES = QBM * QBK * 2;      // 32 KB
constexpr int QH_BYTES = QBN * QBK * 2;      // 16 KB: one k-tile of a chunk
constexpr int QC_BYTES = 2 * QH_BYTES;       // 32 KB: one chunk
constexpr int QLDS = QNS * QA_BYTES + 2 * QC_BYTES;
static_assert(QLDS <= 160 * 1024, "LDS");

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// value of lane (l & ~7) | src(l & 7) for the DPP control CTRL
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                      false));
}
constexpr int DPP_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_HMIR = 0x141;  // row_half_mirror: lane i <-> 7-i of 8
constexpr int dpp_bcast(int j) { return j * 0x55; }  // lane j of the quad

// min / max of a group spread over the 8 lanes of a set (G8) or over the 4
// lanes of a quad
template <bool G8>
__device__ __forceinline__ void reduce_minmax(float& mn, float& mx) {
  mn = fminf(mn, dpp<DPP_XOR1>(mn));
  mx = fmaxf(mx, dpp<DPP_XOR1>(mx));
  mn = fminf(mn, dpp<DPP_XOR2>(mn));
  mx = fmaxf(mx, dpp<DPP_XOR2>(mx));
  if (G8) {
    mn = fminf(mn, dpp<DPP_HMIR>(mn));
    mx = fmaxf(mx, dpp<DPP_HMIR>(mx));
  }
}

// One quantization job of a lane: row r of the tile, channels 8p..8p+7 of
// both k-tile halves h of the chunk (weights wv[h], scales dh[2h + i],
// dhi[2h + i] for channel quarter i).  In three parts, so that the k-tile's
// MFMAs can be spread between them: scaling and local extrema, the group
// reduction and division, then the codes and W_hat of one half.
template <int GS, int QF>
struct QuantJob {
  float u[2][8];
  float mn[2], mx[2], s[2], inv[2];

  __device__ __forceinline__ void scale(const u32x4 (&wv)[2], const f32x4 (&dh)[4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 w = wv[h];
      const f32x4 d0 = dh[2 * h], d1 = dh[2 * h + 1];
      u[h][0] = bf16lo(w.x) * d0.x; u[h][1] = bf16hi(w.x) * d0.y;
      u[h][2] = bf16lo(w.y) * d0.z; u[h][3] = bf16hi(w.y) * d0.w;
      u[h][4] = bf16lo(w.z) * d1.x; u[h][5] = bf16hi(w.z) * d1.y;
      u[h][6] = bf16lo(w.w) * d1.z; u[h][7] = bf16hi(w.w) * d1.w;
      mn[h] = u[h][0];
      mx[h] = u[h][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) {
        mn[h] = fminf(mn[h], u[h][e]);
        mx[h] = fmaxf(mx[h], u[h][e]);
      }
    }
  }

  __device__ __forceinline__ void divide(float Nf, int p) {
    if constexpr (GS == 128) {  // the lane's 16 channels are one group
      mn[0] = fminf(mn[0], mn[1]);
      mx[0] = fmaxf(mx[0], mx[1]);
      reduce_minmax<true>(mn[0], mx[0]);
      mn[1] = mn[0];
      s[0] = qscale<QF>(mn[0], mx[0], Nf);
      inv[0] = s[0] > 0.f ? 1.0f / s[0] : 0.f;
      s[1] = s[0];
      inv[1] = inv[0];
    } else {  // one group per half
      reduce_minmax<GS == 64>(mn[0], mx[0]);
      reduce_minmax<GS == 64>(mn[1], mx[1]);
      // lanes 0 and 1 of each quad divide for halves 0 and 1
      const bool second = p & 1;
      const float mnc = second ? mn[1] : mn[0];
      const float mxc = second ? mx[1] : mx[0];
      const float sc = qscale<QF>(mnc, mxc, Nf);
      const float ic = sc > 0.f ? 1.0f / sc : 0.f;
      s[0] = dpp<dpp_bcast(0)>(sc); inv[0] = dpp<dpp_bcast(0)>(ic);
      s[1] = dpp<dpp_bcast(1)>(sc); inv[1] = dpp<dpp_bcast(1)>(ic);
    }
  }

  // W_hat of half h, 8 bf16
  __device__ __forceinline__ u32x4 dequant(int h, const f32x4 (&dhi)[4], float Nf) const {
    const QGroup g = qgroup_si<QF>(mn[h], s[h], inv[h], Nf);
    float q[8], wq[8];
    qlevels8<QF>(g, u[h], q);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x4 di = dhi[2 * h + (e >> 2)];
      wq[e] = fmaf(s[h], q[e], g.c) * di[e & 3];
    }
    u32x4 o;
    o.x = pack_bf16(wq[0], wq[1]);
    o.y = pack_bf16(wq[2], wq[3]);
    o.z = pack_bf16(wq[4], wq[5]);
    o.w = pack_bf16(wq[6], wq[7]);
    return o;
  }
};

// W_hat of half h, row r, lane p into the chunk at `chunk`
__device__ __forceinline__ void store_what(unsigned char* chunk, int h, int r, int p,
                                           u32x4 o) {
  *(u32x4*)(chunk + h * QH_BYTES + r * 128 + ((p ^ swz(r)) << 4)) = o;
}

template <int GS, int QF>
__device__ __forceinline__ void quant_job(const u32x4 (&wv)[2],
                                          const f32x4 (&dh)[4],
                                          const f32x4 (&dhi)[4], float Nf,
                                          int p, int r, unsigned char* chunk) {
  QuantJob<GS, QF> J;
  J.scale(wv, dh);
  J.divide(Nf, p);
  store_what(chunk, 0, r, p, J.dequant(0, dhi, Nf));
  store_what(chunk, 1, r, p, J.dequant(1, dhi, Nf));
}

// Inputs of one job of a lane, one ring slot: bf16 weights (CB = 0) or
// codes of CB-bit containers with their group's scale and minimum (CB > 0),
// for the two k-tile halves.
template <int CB>
struct JobIn {
  u32x4 w[2];
  unsigned c[2][CB == 8 ? 2 : 1];
  float s[2], m[2];
  f32x4 s4, m4;  // groups of 32: the four groups of the chunk row
};

// Stored codes -> W_hat of half h: bf16((m + s q) D^{-1/2}), the expansion
// of the quantize-once storage ("TTQ: Activation-Aware Test-Time
// Quantization ...", nl summary, Sec. 2: statistics per prompt, weights
// stored quantized), with the float32 operations of the dequantize pass.
template <int CB, int GS, bool F8>
__device__ __forceinline__ u32x4 dequant_half(const JobIn<CB>& J, int h,
                                              const f32x4 (&dhi)[4], int p) {
  float sg, mg;
  if constexpr (GS == 32) {  // group 2h + p/4 of the chunk row
    // (the four values as scalars first: a select between two elements of
    // the ring's vectors made the compiler keep the whole ring in scratch)
    const bool odd = p & 4;
    const float s0 = h ? J.s4.z : J.s4.x, s1 = h ? J.s4.w : J.s4.y;
    const float m0 = h ? J.m4.z : J.m4.x, m1 = h ? J.m4.w : J.m4.y;
    sg = odd ? s1 : s0;
    mg = odd ? m1 : m0;
  } else {
    sg = J.s[h];
    mg = J.m[h];
  }
  float wq[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float qv;
    if constexpr (F8) qv = e4m3_byte(J.c[h][e >> 2], e & 3);
    else if constexpr (CB == 8) qv = (float)((J.c[h][e >> 2] >> ((e & 3) * 8)) & 0xffu);
    else qv = (float)__builtin_amdgcn_ubfe(J.c[h][0], e * CB, CB);
    const f32x4 di = dhi[2 * h + (e >> 2)];
    wq[e] = fmaf(sg, qv, mg) * di[e & 3];
  }
  u32x4 o;
  o.x = pack_bf16(wq[0], wq[1]);
  o.y = pack_bf16(wq[2], wq[3]);
  o.z = pack_bf16(wq[4], wq[5]);
  o.w = pack_bf16(wq[6], wq[7]);
  return o;
}

// CB = 0: quantize bf16 weights with the request's D (path of ttq_linear) in
// format QF; CB = 1, 2, 4, 8: expand stored codes (path of ttq_qmatmul),
// decoded as E4M3 values for QF == QF_FP8 (CB = 8) and as integers otherwise.
template <int GS, int CB, int QF>
__global__ __launch_bounds__(QNW * 64, 1) void k_gemm_q(GemmQArgs a) {
  if (blockIdx.y > 0) {  // product z of a batch
    const int64_t z = blockIdx.y;
    a.X += z * a.sX;
    a.dh += z * a.K1;
    a.dhi += z * a.K1;
    if (a.A2) a.A2 += z * a.sA2;
    a.C += z * a.sC;
  }
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* const sA = smem;
  unsigned char* const sB = smem + QNS * QA_BYTES;

  const int64_t mtiles = (a.M + QBM - 1) / QBM;
  const int64_t ntiles = (a.N + QBN - 1) / QBN;
  const int64_t id = blockIdx.x;
  int64_t ntile, mtile;
  if (ntiles >= 8) {  // token tiles of one weight tile back to back on one XCD
    const int xcd = (int)(id & 7);
    const int64_t j = id >> 3;
    ntile = (j / mtiles) * 8 + xcd;
    mtile = j % mtiles;
  } else {
    ntile = id % ntiles;
    mtile = id / ntiles;
  }
  if (ntile >= ntiles || mtile >= mtiles) return;
  const int64_t m0 = mtile * QBM, n0 = ntile * QBN;
  const int64_t mrows = min((int64_t)QBM, a.M - m0);
  const int64_t nrows = min((int64_t)QBN, a.N - n0);

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float Nf = a.Nf;
  const int nk1 = (int)(a.K1 / QBK);  // even: K1 % 128 == 0
  const int nk2 = a.K2 > 0 ? (int)((a.K2 + QBK - 1) / QBK) : 0;
  const int nk = nk1 + nk2;

  // ---- tile loads straight into LDS (activations, low-rank weights):
  // wave w, instruction j fills rows (w + 8j)*8 .. +8; lane l writes row
  // +l/8, physical chunk l%8 (logical (l%8) ^ swz(row), fixed per lane)
  const int lrow = l >> 3;
  const int lch = (l & 7) ^ swz(w * 8 + lrow);
  const auto rx = make_rsrc(a.X + m0 * a.ldx, (uint32_t)(mrows * a.ldx * 2));
  const auto ra2 = make_rsrc(a.A2 ? a.A2 + m0 * a.lda2 : a.X,
                             a.A2 ? (uint32_t)(mrows * a.lda2 * 2) : 0u);
  const auto rb2 = make_rsrc(a.B2 ? a.B2 + n0 * a.ldb2 : a.X,
                             a.B2 ? (uint32_t)(nrows * a.ldb2 * 2) : 0u);
  // activation tile kt < nk1 (nothing at or past nk1) into stage st; the
  // tile's part of the offset is a scalar, so that no control flow splits
  // the scheduling region of a k-tile
  const int ldx = __builtin_amdgcn_readfirstlane((int)a.ldx);
  const uint32_t ax_lane = (uint32_t)(((w * 8 + lrow) * ldx + lch * 8) * 2);
  auto issue_x = [&](int kt, int st) {
    const uint32_t so = kt < nk1 ? (uint32_t)(kt * QBK * 2) : kOutOfRange;
    unsigned char* dst = sA + st * QA_BYTES + w * 1024;
#pragma unroll
    for (int j = 0; j < QBM / (8 * QNW); ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(dst + j * QNW * 1024), 16,
          ax_lane + so, (uint32_t)(j * 8 * QNW * ldx * 2), 0, 0);
  };
  // low-rank activation tile t (Z, K2 columns) into stage st
  const int lda2 = __builtin_amdgcn_readfirstlane((int)a.lda2);
  auto issue_a2 = [&](int t, int st) {
    const int k0 = t * QBK;
    const bool in = t < nk2 && k0 + lch * 8 < a.K2;
    const uint32_t v =
        in ? (uint32_t)(((w * 8 + lrow) * lda2 + k0 + lch * 8) * 2) : kOutOfRange;
    unsigned char* dst = sA + st * QA_BYTES + w * 1024;
#pragma unroll
    for (int j = 0; j < QBM / (8 * QNW); ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra2, (__attribute__((address_space(3))) void*)(dst + j * QNW * 1024), 16, v,
          (uint32_t)(j * 8 * QNW * lda2 * 2), 0, 0);
  };
  // low-rank weight tile of k-tile kt (>= nk1) into its chunk half
  auto issue_b2 = [&](int kt) {
    const int t = kt - nk1;
    const int ld = __builtin_amdgcn_readfirstlane((int)a.ldb2);
    const int k0 = t * QBK;
    const bool in = t < nk2 && k0 + lch * 8 < a.K2;
    const uint32_t v = in ? (uint32_t)(((w * 8 + lrow) * ld + k0 + lch * 8) * 2)
                          : kOutOfRange;
    unsigned char* dst = sB + ((kt >> 1) & 1) * QC_BYTES + (kt & 1) * QH_BYTES + w * 1024;
#pragma unroll
    for (int j = 0; j < QBN / (8 * QNW); ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb2, (__attribute__((address_space(3))) void*)(dst + j * QNW * 1024), 16, v,
          (uint32_t)(j * 8 * QNW * ld * 2), 0, 0);
  };

  // ---- weight jobs: job q covers row (q & 1)*64 + w*8 + l/8 of chunk q/2,
  // channels 8p..8p+7 of both k-tile halves
  const int p = l & 7;
  const int jrow = w * 8 + (l >> 3);
  const auto rdh = make_rsrc(a.dh, CB == 0 ? (uint32_t)(a.K1 * 4) : 0u);
  const auto rdhi = make_rsrc(a.dhi, (uint32_t)(a.K1 * 4));
  // lane parts of the offsets; the job's part is a scalar (out of range past
  // the weights, so that every k-tile issues the same number of loads)
  const uint32_t doff = (uint32_t)(p * 32);
  auto load_job = [&](int q, JobIn<CB>& J) {
    const bool in = q < nk1;
    if constexpr (CB == 0) {
      const auto rw = make_rsrc(a.W + n0 * a.ldw, (uint32_t)(nrows * a.ldw * 2));
      const int ldw = __builtin_amdgcn_readfirstlane((int)a.ldw);
      const uint32_t woff = (uint32_t)((jrow * ldw + p * 8) * 2);
      const uint32_t so = in ? (uint32_t)(((q & 1) * 64 * ldw + (q >> 1) * 128) * 2)
                             : kOutOfRange;
#pragma unroll
      for (int h = 0; h < 2; ++h) J.w[h] = buf_load16(rw, woff + so + h * 128, 0);
    } else {
      const int rb = __builtin_amdgcn_readfirstlane((int)a.row_bytes);
      const int G = __builtin_amdgcn_readfirstlane((int)a.G);
      const auto rc = make_rsrc(a.packed + n0 * a.row_bytes, (uint32_t)(nrows * a.row_bytes));
      const auto rs = make_rsrc(a.s + n0 * a.G, (uint32_t)(nrows * a.G * 4));
      const auto rm = make_rsrc(a.m + n0 * a.G, (uint32_t)(nrows * a.G * 4));
      // codes: channel c of row r at byte r * row_bytes + c * CB / 8
      const uint32_t so = in ? (uint32_t)((q & 1) * 64 * rb + (q >> 1) * 16 * CB) : kOutOfRange;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t off = (uint32_t)(jrow * rb + p * CB + h * 8 * CB) + so;
        if constexpr (CB == 8) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0);
          J.c[h][0] = v[0];
          J.c[h][1] = v[1];
        } else if constexpr (CB == 4) {
          J.c[h][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, off, 0, 0);
        } else if constexpr (CB == 2) {
          J.c[h][0] = __builtin_amdgcn_raw_buffer_load_b16(rc, off, 0, 0);
        } else {
          J.c[h][0] = __builtin_amdgcn_raw_buffer_load_b8(rc, off, 0, 0);
        }
      }
      // group of channel (q/2)*128 + 64h + 8p: one group for both halves
      // (GS >= 128), two adjacent ones (64: one 8-byte load), or groups
      // 2h + p/4 of four (32)
      const int gq = GS >= 128 ? (q >> 1) * 128 / GS : (q >> 1) * (128 / GS);
      const uint32_t sso = in ? (uint32_t)(((q & 1) * 64 * G + gq) * 4) : kOutOfRange;
      if constexpr (GS >= 128) {
        const uint32_t off = (uint32_t)(jrow * G * 4) + sso;
        J.s[0] = J.s[1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        J.m[0] = J.m[1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm, off, 0, 0));
      } else if constexpr (GS == 64) {
        const uint32_t off = (uint32_t)(jrow * G * 4) + sso;
        // (the whole vector is reinterpreted: a bit_cast of one lane of the
        // loaded vector was compiled into a one-dword load of lane 0)
        typedef __attribute__((ext_vector_type(2))) float f32x2;
        const f32x2 sv = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
        const f32x2 mv = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rm, off, 0, 0));
        J.s[0] = sv.x;
        J.s[1] = sv.y;
        J.m[0] = mv.x;
        J.m[1] = mv.y;
      } else {
        const uint32_t off = (uint32_t)(jrow * G * 4) + sso;
        J.s4 = __builtin_bit_cast(f32x4, buf_load16(rs, off, 0));
        J.m4 = __builtin_bit_cast(f32x4, buf_load16(rm, off, 0));
      }
    }
  };
  auto load_dh = [&](int c, f32x4 (&dv)[4], f32x4 (&iv)[4]) {
    const uint32_t so = 2 * c < nk1 ? (uint32_t)(c * 512) : kOutOfRange;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t off = doff + (uint32_t)(h * 256 + i * 16) + so;
        if constexpr (CB == 0)
          dv[2 * h + i] = __builtin_bit_cast(f32x4, buf_load16(rdh, off, 0));
        iv[2 * h + i] = __builtin_bit_cast(f32x4, buf_load16(rdhi, off, 0));
      }
  };
  // loads per k-tile: activation tile, scales of a chunk (even k-tiles), job
  constexpr int NA = QBM / (8 * QNW);
  constexpr int ND = CB == 0 ? 8 : 4;
  constexpr int NJ = CB == 0 ? 2 : 4;

  // ---- MFMA part: wave (wm, wn) owns 64 tokens x 64 weight rows
  const int wm = w >> 1, wn = w & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int fs = swz(l & 15);
  const int fh = l >> 5;
  const int arow = (wm * 64 + (l & 31)) * 128;
  const int brow = (wn * 64 + (l & 31)) * 128;
  auto read_frags = [&](const unsigned char* sa, const unsigned char* sb, int kk,
                        u32x4 (&fa)[2], u32x4 (&fb)[2]) {
    const int off = (((kk << 1) | fh) ^ fs) * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = *(const u32x4*)(sb + brow + j * 4096 + off);
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = *(const u32x4*)(sa + arow + i * 4096 + off);
  };
  auto mfmas = [&](const u32x4 (&fa)[2], const u32x4 (&fb)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]),
            acc[i][j], 0, 0, 0);
  };
  // the four MFMA steps of one k-tile
  auto ktile = [&](const unsigned char* sa, const unsigned char* sb) {
    u32x4 fa[2][2], fb[2][2];
    read_frags(sa, sb, 0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) read_frags(sa, sb, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      mfmas(fa[kk & 1], fb[kk & 1]);
    }
  };

  // ---- prologue: chunk 0 ready, activation tiles 0, 1 and the loads of
  // jobs 2..4 and of the scales of chunk 1 in flight
  JobIn<CB> ring[4];
  f32x4 dhv[2][4], dhiv[2][4];
  // one job into the chunk buffer
  auto job = [&](const JobIn<CB>& J, int ds, int r) {
    unsigned char* chunk = sB + ds * QC_BYTES;
    if constexpr (CB == 0) {
      quant_job<GS, QF>(J.w, dhv[ds], dhiv[ds], Nf, p, r, chunk);
    } else {
      store_what(chunk, 0, r, p, dequant_half<CB, GS, QF == QF_FP8>(J, 0, dhiv[ds], p));
      store_what(chunk, 1, r, p, dequant_half<CB, GS, QF == QF_FP8>(J, 1, dhiv[ds], p));
    }
  };
  // (issue order fixed: the first wait below counts on it, and the weights
  // of jobs 2 and 3 are as old as those of later jobs at their use)
  load_dh(0, dhv[0], dhiv[0]);
  load_job(0, ring[0]);
  load_job(1, ring[1]);
  load_job(2, ring[2]);
  load_job(3, ring[3]);
  __builtin_amdgcn_sched_barrier(0);
  load_dh(1, dhv[1], dhiv[1]);
  __builtin_amdgcn_sched_barrier(0);
  issue_x(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_x(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  job(ring[0], 0, jrow);
  job(ring[1], 0, 64 + jrow);
  __builtin_amdgcn_sched_barrier(0);
  load_job(4, ring[0]);

  int sta = 0;  // activation stage of k-tile kt
  // k-tile kt < nk1: wait for its activation tile, run its MFMAs and the job
  // kt + 2 (chunk kt/2 + 1; the jobs nk1, nk1 + 1 past the weights write
  // zeros into a chunk that the main loop does not read), then issue the
  // loads two (activations) and three (weights) k-tiles ahead.  POS = kt % 4
  // fixes the register sets: job q in ring slot q % 4, scales of chunk c in
  // set c % 2.
  auto step = [&](int kt, auto pos_c) {
    constexpr int POS = decltype(pos_c)::value;
    constexpr int QS = (POS + 2) & 3;          // ring slot of job kt + 2
    constexpr int DS = (QS >> 1) & 1;          // its scale set and chunk
    // Loads of k-tile kt in issue order: [activation tile: NA] then, in any
    // order, [scales of a chunk: ND, even kt] [job: NJ].  The activation tile
    // of kt (issued in k-tile kt - 2) is followed by at least NA + ND + 2 NJ
    // loads (NA + NJ in the prologue for tile 0).
    if (kt == 0) wait_vm<NA + NJ>();
    else wait_vm<NA + ND + 2 * NJ>();
    lds_barrier();
    const unsigned char* sa = sA + sta * QA_BYTES;
    const unsigned char* sb =
        sB + ((POS >> 1) & 1) * QC_BYTES + (POS & 1) * QH_BYTES;
    // The four MFMA steps with the job's parts between them; fragment reads
    // one step ahead.  LDS writes (weights, direct loads) come after the last
    // fragment read.
    u32x4 fa[2][2], fb[2][2];
    u32x4 o0, o1;
    if constexpr (CB == 0) {
      QuantJob<GS, QF> J;
      read_frags(sa, sb, 0, fa[0], fb[0]);
      J.scale(ring[QS].w, dhv[DS]);
      __builtin_amdgcn_sched_barrier(0);
      read_frags(sa, sb, 1, fa[1], fb[1]);
      mfmas(fa[0], fb[0]);
      J.divide(Nf, p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 9, 1);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      read_frags(sa, sb, 2, fa[0], fb[0]);
      mfmas(fa[1], fb[1]);
      o0 = J.dequant(0, dhiv[DS], Nf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 13, 2);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      read_frags(sa, sb, 3, fa[1], fb[1]);
      mfmas(fa[0], fb[0]);
      o1 = J.dequant(1, dhiv[DS], Nf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 13, 3);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(fa[1], fb[1]);
    } else {
      read_frags(sa, sb, 0, fa[0], fb[0]);
      read_frags(sa, sb, 1, fa[1], fb[1]);
      mfmas(fa[0], fb[0]);
      o0 = dequant_half<CB, GS, QF == QF_FP8>(ring[QS], 0, dhiv[DS], p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 1);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      read_frags(sa, sb, 2, fa[0], fb[0]);
      mfmas(fa[1], fb[1]);
      o1 = dequant_half<CB, GS, QF == QF_FP8>(ring[QS], 1, dhiv[DS], p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 2);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      read_frags(sa, sb, 3, fa[1], fb[1]);
      mfmas(fa[0], fb[0]);
      mfmas(fa[1], fb[1]);
    }
    unsigned char* chunk = sB + DS * QC_BYTES;
    const int r = (QS & 1) * 64 + jrow;
    store_what(chunk, 0, r, p, o0);
    store_what(chunk, 1, r, p, o1);
    const int st2 = sta == 0 ? 2 : sta - 1;  // stage of kt + 2
    issue_x(kt + 2, st2);
    __builtin_amdgcn_sched_barrier(0);
    if (POS % 2 == 0) load_dh(kt / 2 + 2, dhv[(POS / 2) & 1], dhiv[(POS / 2) & 1]);
    load_job(kt + 5, ring[(POS + 1) & 3]);
    sta = sta == QNS - 1 ? 0 : sta + 1;
  };
  int kt = 0;
  for (; kt + 4 <= nk1; kt += 4) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
    step(kt + 2, std::integral_constant<int, 2>{});
    step(kt + 3, std::integral_constant<int, 3>{});
  }
  if (kt < nk1) {  // nk1 is even
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
  }

  // low-rank segment, one chunk (two k-tiles) at a time
  for (int t = 0; t < nk2; t += 2) {
    kt = nk1 + t;
    lds_barrier();  // the chunk's buffer and the stages are no longer used
    issue_b2(kt);
    issue_b2(kt + 1);
    issue_a2(t, kt % QNS);
    issue_a2(t + 1, (kt + 1) % QNS);
    wait_vm<0>();
    lds_barrier();
    const unsigned char* sb = sB + ((kt >> 1) & 1) * QC_BYTES;
    ktile(sA + (kt % QNS) * QA_BYTES, sb);
    if (t + 1 < nk2) ktile(sA + ((kt + 1) % QNS) * QA_BYTES, sb + QH_BYTES);
  }
  // loads issued past the last tile read nothing but still write LDS / VGPRs
  wait_vm<0>();

  // C layout of a 32x32 MFMA tile: lane l holds column l%32 and rows
  // 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
        const int64_t n = n0 + wn * 64 + j * 32 + (l & 31);
        if (m < a.M && n < a.N) a.C[m * a.ldc + n] = acc[i][j][r];
      }
}

}  // namespace

bool gemm_q_supported(int64_t K1, int group, int cb) {
  if (K1 <= 0 || K1 % 128 != 0) return false;
  if (group == 32 || group == 64 || group == 128) return true;
  return cb > 0 && group == 256;  // no group reduction when expanding codes
}

namespace {

template <int GS, int CB, int QF>
hipError_t launch_gq(const GemmQArgs& a, dim3 grid, const Launch& L) {
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(k_gemm_q<GS, CB, QF>),
      hipFuncAttributeMaxDynamicSharedMemorySize, QLDS);
  if (attr != hipSuccess) return attr;
  return ext_launch(k_gemm_q<GS, CB, QF>, grid, dim3(QNW * 64), QLDS, L, a);
}

template <int CB, int QF>
hipError_t launch_gq_cb(const GemmQArgs& a, int group, dim3 grid, const Launch& L) {
  switch (group) {
    case 32: return launch_gq<32, CB, QF>(a, grid, L);
    case 64: return launch_gq<64, CB, QF>(a, grid, L);
    case 128: return launch_gq<128, CB, QF>(a, grid, L);
    case 256:
      if constexpr (CB > 0) return launch_gq<256, CB, QF>(a, grid, L);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_q(const GemmQArgs& a, int group, int cb, const Launch& L) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!gemm_q_supported(a.K1, group, cb) || !a.C) return hipErrorInvalidValue;
  if (cb > 0 && (!a.packed || !a.s || !a.m || a.row_bytes * 8 != a.K1 * cb))
    return hipErrorInvalidValue;
  const int64_t mtiles = (a.M + QBM - 1) / QBM;
  const int64_t ntiles = (a.N + QBN - 1) / QBN;
  const int64_t nblk =
      ntiles >= 8 ? ((ntiles + 7) / 8) * 8 * mtiles : ntiles * mtiles;
  const unsigned nb = a.batch > 1 ? (unsigned)a.batch : 1u;
  const dim3 grid((unsigned)nblk, nb);
  if (cb == 0) {
    switch (a.qf) {
      case QF_ASYM: return launch_gq_cb<0, QF_ASYM>(a, group, grid, L);
      case QF_SYM: return launch_gq_cb<0, QF_SYM>(a, group, grid, L);
      case QF_INTZP: return launch_gq_cb<0, QF_INTZP>(a, group, grid, L);
      case QF_FP8: return launch_gq_cb<0, QF_FP8>(a, group, grid, L);
      default: return hipErrorInvalidValue;
    }
  }
  // stored codes: the integer formats share one decoding (u_hat = m + s q
  // with the stored offset m); E4M3 codes are 8-bit
  if (a.qf == QF_FP8)
    return cb == 8 ? launch_gq_cb<8, QF_FP8>(a, group, grid, L) : hipErrorInvalidValue;
  switch (cb) {
    case 1: return launch_gq_cb<1, QF_ASYM>(a, group, grid, L);
    case 2: return launch_gq_cb<2, QF_ASYM>(a, group, grid, L);
    case 4: return launch_gq_cb<4, QF_ASYM>(a, group, grid, L);
    case 8: return launch_gq_cb<8, QF_ASYM>(a, group, grid, L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttq
