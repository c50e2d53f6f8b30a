// Contraction of new activations with stored packed codes (quantize once
// per prompt, then decode): the deployed form of TTQ keeps the b-bit codes,
// the per-group (s, min) and D^{-1/2} of the prompt and contracts later
// tokens with them ("TTQ: Activation-Aware Test-Time Quantization ...", nl
// summary, Sec. 2-3; zh summary, Sec. 3-4: speed from low-bit weights,
// whose transfer is the bottleneck).
//
//   y_i = sum_g  s_ig * sum_{j in g} q_ij x'_j  +  m_ig * sum_{j in g} x'_j
//         + B_i . z,           x' = x D^{-1/2},  z = A x
//
// which is ((m + s q) D^{-1/2}) x regrouped so that each code is one
// multiply-add on the VALU.
//
// k_qgemv (one token): a workgroup of 8 waves owns 16 rows, two per wave.
// Each wave first issues the first loads of its two rows of codes (one
// 16-byte load per lane covers 128 / CB codes, a wave load 1 KiB of a row)
// and their (s, min); while they are in flight the workgroup puts x'
// (float32) and the per-slice sums of x' in LDS.  Later loads of a row are
// issued as earlier ones are consumed.  A lane's slice of SUB = min(128 /
// CB, GS) channels lies in one group; its partial product is scaled by that
// group's s and its slice sum by m.  Rows are reduced across the wave in a
// fixed butterfly order (deterministic).
//
// k_dequant (more tokens): expands the codes to W_hat = bf16((m + s q)
// D^{-1/2}), the operand of the large-tile GEMM.
#include "ttq_internal.h"

namespace ttq {

namespace {

constexpr int QW = 8;    // waves per workgroup
constexpr int QRPW = 2;  // rows per wave
constexpr int QNB = 4;   // 1 KiB loads in flight per row

// float value of code j (0 .. 128/CB - 1) of a 16-byte piece (F8: E4M3
// codes, CB = 8)
template <int CB, bool F8>
__device__ __forceinline__ float code_at(const u32x4& v, int j) {
  static_assert(!F8 || CB == 8, "E4M3 codes are 8 bits wide");
  constexpr int PER = 32 / CB;  // codes per 32-bit word
  const unsigned w = j / PER < 2 ? (j / PER == 0 ? v.x : v.y)
                                 : (j / PER == 2 ? v.z : v.w);
  const int sh = (j % PER) * CB;
  if constexpr (F8) return e4m3_byte(w, j % PER);
  if (CB == 8) return (float)((w >> sh) & 0xffu);
  return (float)__builtin_amdgcn_ubfe(w, sh, CB);
}

template <int CB, int GS, bool F8>
__global__ __launch_bounds__(QW * 64) void k_qgemv(QGemvArgs a) {
  constexpr int VPL = 128 / CB;                 // codes per lane per load
  constexpr int SUB = VPL < GS ? VPL : GS;      // channels per slice
  constexpr int NSB = VPL / SUB;                // slices per load
  constexpr int CPL = 64 * VPL;                 // channels per wave load
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int64_t d = a.d;
  const int64_t dpad = (d + CPL - 1) / CPL * CPL;
  float* xp = lds;               // [dpad] x', in read order
  float* sxs = lds + dpad;       // [dpad / SUB] slice sums of x', in read order

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t row0 = ((int64_t)blockIdx.x * QW + w) * QRPW;
  const int nld = (int)((a.row_bytes + 1023) / 1024);  // loads per row

  // x' = x * D^{-1/2} (zero past d) and its slice sums go to LDS, laid out
  // for the reads of the main loop: lane l of every wave reads channels
  // k*CPL + l*VPL + [0, VPL) of load k, so value i of that run sits at
  // float ((k*VPL/4 + i/4)*64 + l)*4 + i%4 and the sum of slice sb at
  // (k*NSB + sb)*64 + l (consecutive lanes, consecutive 16 bytes: no bank
  // conflicts).  Each thread prepares 4 channels per step; the SUB/4
  // threads of one slice are adjacent lanes and add their parts with
  // xor-shuffles in a fixed order.  The activation loads of the first two
  // steps are issued before the code stream, so that x' is ready as soon
  // as they return.
  constexpr int LPS = SUB / 4;                  // lanes per slice
  const int64_t nitem = dpad / 4;               // multiple of 256
  // Bounded buffer loads: channels past d read zeros with no branch.  (A
  // guarded load made the compiler wait for it before the code stream was
  // requested, putting the two latencies in series.)
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.X, (uint32_t)(d * 2));
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.dhi, (uint32_t)(d * 4));
  auto xload = [&](int64_t it, u32x2& xv, f32x4& h) {
    const int64_t q = it / LPS, i = (it % LPS) * 4;
    const int64_t ln = q & 63, ks = q >> 6;
    const int64_t c = (ks / NSB) * CPL + ln * VPL + (ks % NSB) * SUB + i;
    xv = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(xr, (uint32_t)(c * 2), 0, 0));
    h = __builtin_bit_cast(f32x4, buf_load16(hr, (uint32_t)(c * 4), 0));
  };
  auto xstore = [&](int64_t it, const u32x2& xv, const f32x4& h) {
    const int64_t q = it / LPS, i = (it % LPS) * 4;
    const int64_t ln = q & 63, ks = q >> 6;
    const int64_t k = ks / NSB, sb = ks % NSB;
    const f32x4 xv4 = {bf16lo(xv.x) * h.x, bf16hi(xv.x) * h.y,
                       bf16lo(xv.y) * h.z, bf16hi(xv.y) * h.w};
    *(f32x4*)(xp + ((k * (VPL / 4) + (sb * SUB + i) / 4) * 64 + ln) * 4) = xv4;
    float sum = (xv4.x + xv4.y) + (xv4.z + xv4.w);
#pragma unroll
    for (int off = LPS / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (i == 0) sxs[ks * 64 + ln] = sum;
  };
  u32x2 xv0, xv1;
  f32x4 h0, h1;
  const int64_t it0 = tid, it1 = tid + QW * 64;  // wave-uniform validity
  xload(it0, xv0, h0);   // (items past the padded range read zeros)
  xload(it1, xv1, h1);
  __builtin_amdgcn_sched_barrier(0);

  // A ring of QNB loads per row: load k of a row lives in slot k % QNB and
  // is replaced by load k + QNB as soon as it has been consumed.  Rows past
  // d_out read an empty buffer (zeros) and are not stored.
  u32x4 v[QRPW][QNB];
  float sg[QRPW][QNB][NSB], mg[QRPW][QNB][NSB];
  __amdgpu_buffer_rsrc_t cr[QRPW];
  int64_t srow[QRPW];
#pragma unroll
  for (int rr = 0; rr < QRPW; ++rr) {
    const int64_t row = row0 + rr;
    const bool rlive = row < a.d_out;
    cr[rr] = make_rsrc(a.packed + (rlive ? row : 0) * a.row_bytes,
                       rlive ? (uint32_t)a.row_bytes : 0u);
    srow[rr] = (rlive ? row : 0) * a.G;
  }
  // Every fetch is issued, with no branch: a load past the row reads zeros
  // and its scale index is clamped to a valid one.  With the loads in
  // branches the compiler's wait counts at the joins became conservative
  // (the x' prologue waited for the whole code stream).
  auto fetch = [&](int rr, int slot, int k) {
    const bool live = k < nld;  // uniform
    v[rr][slot] = buf_load16(cr[rr], (uint32_t)(l * 16), live ? (uint32_t)k * 1024 : kOutOfRange);
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      const int64_t cs = (int64_t)k * CPL + (int64_t)l * VPL + sb * SUB;
      const int64_t gi = srow[rr] + (live && cs < d ? cs / GS : 0);
      sg[rr][slot][sb] = a.s[gi];
      mg[rr][slot][sb] = a.m[gi];
    }
  };
#pragma unroll
  for (int rr = 0; rr < QRPW; ++rr)
#pragma unroll
    for (int j = 0; j < QNB; ++j) fetch(rr, j, j);
  __builtin_amdgcn_sched_barrier(0);

  if (it0 < nitem) xstore(it0, xv0, h0);
  if (it1 < nitem) xstore(it1, xv1, h1);
  for (int64_t it = tid + 2 * QW * 64; it < nitem; it += QW * 64) {
    u32x2 xv;
    f32x4 h;
    xload(it, xv, h);
    xstore(it, xv, h);
  }
  __syncthreads();

#pragma unroll
  for (int rr = 0; rr < QRPW; ++rr) {
    const int64_t row = row0 + rr;
    if (row >= a.d_out) break;  // wave-uniform
    float acc = 0.f;
    for (int kb = 0; kb < nld; kb += QNB) {
#pragma unroll
      for (int j = 0; j < QNB; ++j) {
        const int k = kb + j;
        if (k >= nld) break;  // uniform
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
          // slices past d add nothing (a select, not a branch: padding
          // bytes of a row need not hold finite codes)
          const bool in_d = (int64_t)k * CPL + (int64_t)l * VPL + sb * SUB < d;
          float P0 = 0.f, P1 = 0.f, P2 = 0.f, P3 = 0.f;
#pragma unroll
          for (int i = 0; i < SUB; i += 4) {
            const f32x4 xq = *(const f32x4*)(
                xp + ((k * (VPL / 4) + (sb * SUB + i) / 4) * 64 + l) * 4);
            P0 = fmaf(code_at<CB, F8>(v[rr][j], sb * SUB + i + 0), xq.x, P0);
            P1 = fmaf(code_at<CB, F8>(v[rr][j], sb * SUB + i + 1), xq.y, P1);
            P2 = fmaf(code_at<CB, F8>(v[rr][j], sb * SUB + i + 2), xq.z, P2);
            P3 = fmaf(code_at<CB, F8>(v[rr][j], sb * SUB + i + 3), xq.w, P3);
          }
          const float P = in_d ? (P0 + P1) + (P2 + P3) : 0.f;
          acc = fmaf(sg[rr][j][sb], P,
                     fmaf(mg[rr][j][sb], sxs[(k * NSB + sb) * 64 + l], acc));
        }
        fetch(rr, j, k + QNB);
      }
    }
    // static low-rank term: + B[row, :] . z
    for (int k = l; k < a.rank; k += 64)
      acc = fmaf(__uint_as_float((unsigned)a.Blr[row * a.rank + k] << 16),
                 __uint_as_float((unsigned)a.Z[k] << 16), acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (l == 0) a.Y[row] = acc;
  }
}

template <int CB, int GS, bool F8>
__global__ __launch_bounds__(256) void k_dequant(DequantArgs a) {
  constexpr int VPL = 128 / CB;
  const int64_t lanes_per_row = a.row_bytes / 16;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = id / lanes_per_row, piece = id % lanes_per_row;
  if (row >= a.d_out) return;
  const u32x4 v = *(const u32x4*)(a.packed + row * a.row_bytes + piece * 16);
  const int64_t c0 = piece * VPL;
  bf16_t* out = a.What + row * a.d + c0;
#pragma unroll
  for (int j = 0; j < VPL; j += 8) {
    if (c0 + j >= a.d) break;
    const int64_t g = (c0 + j) / GS;
    const float sg = a.s[row * a.G + g], mg = a.m[row * a.G + g];
    const f32x4 h0 = *(const f32x4*)(a.dhi + c0 + j);
    const f32x4 h1 = *(const f32x4*)(a.dhi + c0 + j + 4);
    const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
    float wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[i] = fmaf(sg, code_at<CB, F8>(v, j + i), mg) * hv[i];
    *(u32x4*)(out + j) = u32x4{pack_bf16(wv[0], wv[1]), pack_bf16(wv[2], wv[3]),
                               pack_bf16(wv[4], wv[5]), pack_bf16(wv[6], wv[7])};
  }
}

}  // namespace

size_t qgemv_lds_bytes(int64_t d, int cb, int group) {
  const int64_t vpl = 128 / cb, cpl = 64 * vpl;
  const int64_t sub = vpl < group ? vpl : group;
  const int64_t dpad = (d + cpl - 1) / cpl * cpl;
  return (size_t)(dpad + dpad / sub) * sizeof(float);
}

hipError_t launch_qgemv(const QGemvArgs& a, int group, int cb,
                        const Launch& L) {
  const int64_t rows = (int64_t)QW * QRPW;  // per workgroup
  const int64_t nblk = (a.d_out + rows - 1) / rows;
  if (nblk == 0) return hipSuccess;
  if (a.row_bytes % 16 != 0) return hipErrorInvalidValue;
  const uint32_t lds = (uint32_t)qgemv_lds_bytes(a.d, cb, group);
  const dim3 grid((unsigned)nblk), blk(QW * 64);
#define TTQ_QGEMV_GS(CBV, F8)                                                 \
  switch (group) {                                                            \
    case 32: return ext_launch(k_qgemv<CBV, 32, F8>, grid, blk, lds, L, a);   \
    case 64: return ext_launch(k_qgemv<CBV, 64, F8>, grid, blk, lds, L, a);   \
    case 128: return ext_launch(k_qgemv<CBV, 128, F8>, grid, blk, lds, L, a); \
    case 256: return ext_launch(k_qgemv<CBV, 256, F8>, grid, blk, lds, L, a); \
    default: return hipErrorInvalidValue;                                     \
  }
  if (a.qf == QF_FP8) {
    if (cb != 8) return hipErrorInvalidValue;
    TTQ_QGEMV_GS(8, true)
  }
  switch (cb) {
    case 1: TTQ_QGEMV_GS(1, false)
    case 2: TTQ_QGEMV_GS(2, false)
    case 4: TTQ_QGEMV_GS(4, false)
    case 8: TTQ_QGEMV_GS(8, false)
    default: return hipErrorInvalidValue;
  }
#undef TTQ_QGEMV_GS
}

hipError_t launch_dequant(const DequantArgs& a, int group, int cb,
                          const Launch& L) {
  if (a.row_bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t threads = a.d_out * (a.row_bytes / 16);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256)), blk(256);
#define TTQ_DEQ_GS(CBV, F8)                                                   \
  switch (group) {                                                            \
    case 32: return ext_launch(k_dequant<CBV, 32, F8>, grid, blk, 0, L, a);   \
    case 64: return ext_launch(k_dequant<CBV, 64, F8>, grid, blk, 0, L, a);   \
    case 128: return ext_launch(k_dequant<CBV, 128, F8>, grid, blk, 0, L, a); \
    case 256: return ext_launch(k_dequant<CBV, 256, F8>, grid, blk, 0, L, a); \
    default: return hipErrorInvalidValue;                                     \
  }
  if (a.qf == QF_FP8) {
    if (cb != 8) return hipErrorInvalidValue;
    TTQ_DEQ_GS(8, true)
  }
  switch (cb) {
    case 1: TTQ_DEQ_GS(1, false)
    case 2: TTQ_DEQ_GS(2, false)
    case 4: TTQ_DEQ_GS(4, false)
    case 8: TTQ_DEQ_GS(8, false)
    default: return hipErrorInvalidValue;
  }
#undef TTQ_DEQ_GS
}

}  // namespace ttq
