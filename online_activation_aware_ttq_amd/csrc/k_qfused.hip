// Contraction of a few later tokens (2..128) with stored packed codes on the
// gfx950 matrix cores: the quantize-once counterpart of the fused one-pass
// kernel ("TTQ: Activation-Aware Test-Time Quantization ...", nl summary,
// Sec. 2-3; zh summary, Sec. 3-4: the codes, (s, min) and D^{-1/2} are kept
// from the prompt, and moving low-bit weights is what makes it fast).
//
//   Y[t,i] = sum_g  s_ig * sum_{j in g} q_ij x'_tj  +  m_ig * sum_{j in g} x'_tj
//
// with x' = x D^{-1/2} from the stored D^{-1/2}.  The statistics kernel, in
// its stored-D^{-1/2} mode, writes x' (for T <= 16 fp16 scaled by a power of
// two per group and token, with the inverse factors, as for the one-pass
// kernel; one bf16 plane above; MFMA fragment order) and the per-token group
// sums, in
// the layout the one-pass kernel reads; this kernel streams the codes instead
// of bf16 weights.  The work split is that of the one-pass kernel: 8 or 16
// waves own 16 weight rows and stride over the groups, each with the codes
// and x' of its next group in flight.  Lane l holds row l & 15 and lane
// quarter l >> 4 a contiguous quarter of each group (8 channels per MFMA
// step; x' in the quarter fragment order), i.e. GS/32 * CB contiguous bytes
// of the packed row per group: one wide load.
//
// Codes become the B operand exactly: for containers of up to 4 bits the
// value 128 + q (bf16 bits 0x4300 | q, one byte permute per pair; in fp16 at
// T <= 16, 1024 + q, bits 0x6400 | q), whose extra bias * sum(x') is taken
// out with the minimum term:
//   s * sum (bias + q) x' + (m - bias s) * sum x';
// for 8-bit containers q itself (converted through float32).
#include "ttq_internal.h"

namespace ttq {

namespace {

// waves per workgroup: 16 where the registers allow (more groups in flight
// per CU; the work per group is small), else 8 (also for the E4M3 decoding,
// which needs more registers per code)
template <int NTB, int GS, bool F8>
constexpr int qf_waves() {
  return (NTB <= 2 && GS <= 128 && !F8) ? 16 : 8;
}

// 8 codes of CB bits, low bits first in `raw` -> 4 bf16 pairs (see above),
// or with H16 4 fp16 pairs: 1024 + q (fp16 bits 0x6400 | q) for containers
// of up to 4 bits, q itself for 8-bit containers
template <int CB, bool F8, bool H16 = false>
__device__ __forceinline__ u32x4 codes_operand(u32x2 raw) {
  static_assert(!F8 || CB == 8, "E4M3 codes are 8 bits wide");
  constexpr unsigned OR = H16 ? 0x64006400u : 0x43004300u;
  if (CB == 8) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (F8) {
        f[i] = e4m3_byte(raw.x, i);
        f[4 + i] = e4m3_byte(raw.y, i);
      } else {
        f[i] = (float)((raw.x >> (8 * i)) & 0xFFu);
        f[4 + i] = (float)((raw.y >> (8 * i)) & 0xFFu);
      }
    }
    if constexpr (H16) {  // exact in fp16 (integers up to 255, E4M3 values)
      return u32x4{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(f[0], f[1])),
                   __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(f[2], f[3])),
                   __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(f[4], f[5])),
                   __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(f[6], f[7]))};
    }
    // the high halves of the floats (exact: at most 8 significant bits, or
    // the 4 of an E4M3 value)
    return u32x4{__builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u),
                 __builtin_amdgcn_perm(__float_as_uint(f[3]), __float_as_uint(f[2]), 0x07060302u),
                 __builtin_amdgcn_perm(__float_as_uint(f[5]), __float_as_uint(f[4]), 0x07060302u),
                 __builtin_amdgcn_perm(__float_as_uint(f[7]), __float_as_uint(f[6]), 0x07060302u)};
  } else if (CB == 4) {
    // even codes in the bytes of lo, odd codes in the bytes of hi; pair k =
    // bytes {lo.k, 0, hi.k, 0} (selector 0x0c: zero byte), then | 0x4300
    const unsigned lo = raw.x & 0x0F0F0F0Fu, hi = (raw.x >> 4) & 0x0F0F0F0Fu;
    return u32x4{__builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | OR,
                 __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | OR,
                 __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | OR,
                 __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | OR};
  } else {
    constexpr unsigned M = (1u << CB) - 1u;
    unsigned p[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned q0 = (raw.x >> (2 * k * CB)) & M;
      const unsigned q1 = (raw.x >> ((2 * k + 1) * CB)) & M;
      p[k] = (q0 | (q1 << 16)) | OR;
    }
    return u32x4{p[0], p[1], p[2], p[3]};
  }
}

// A lane's codes of one group: its contiguous quarter of the group, NB =
// GS/32 * CB bytes, fetched with the widest loads that tile it.
template <int CB, int GS>
struct GroupCodes {
  static constexpr int NB = GS / 32 * CB;
  unsigned w[NB >= 4 ? NB / 4 : 1];
};

template <int CB, int GS>
__device__ __forceinline__ void load_codes(GroupCodes<CB, GS>& c,
                                           __amdgpu_buffer_rsrc_t r,
                                           uint32_t voff, uint32_t soff) {
  constexpr int NB = GroupCodes<CB, GS>::NB;
  if constexpr (NB >= 16) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const u32x4 v = buf_load16(r, voff + i * 16, soff);
      c.w[4 * i] = v.x; c.w[4 * i + 1] = v.y; c.w[4 * i + 2] = v.z; c.w[4 * i + 3] = v.w;
    }
  } else if constexpr (NB == 8) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    c.w[0] = v[0];
    c.w[1] = v[1];
  } else if constexpr (NB == 4) {
    c.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  } else if constexpr (NB == 2) {
    c.w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  } else {
    c.w[0] = __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
  }
}

// the 8 codes (CB bytes) of MFMA step k, low bits first
template <int CB, int GS>
__device__ __forceinline__ u32x2 step_codes(const GroupCodes<CB, GS>& c, int k) {
  if (CB == 8) return u32x2{c.w[2 * k], c.w[2 * k + 1]};
  if (CB == 4) return u32x2{c.w[k], 0u};
  if (CB == 2) return u32x2{(c.w[k / 2] >> (16 * (k % 2))) & 0xFFFFu, 0u};
  return u32x2{(c.w[k / 4] >> (8 * (k % 4))) & 0xFFu, 0u};
}

template <int CB, int NTB, int GS, bool F8>
__global__ __launch_bounds__((qf_waves<NTB, GS, F8>() * 64)) void k_qfused(QFusedArgs a) {
  constexpr int QF_W = qf_waves<NTB, GS, F8>();
  constexpr int NKS = GS / 32;
  constexpr bool XF16 = (NTB == 1);   // T <= 16: scaled fp16 operands
  constexpr float BIAS = CB == 8 ? 0.f : (XF16 ? 1024.f : 128.f);
  __shared__ float red[QF_W][NTB * 4][64];

  const int64_t rb = blockIdx.x;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = l & 15, qd = l >> 4;
  const int64_t row = rb * 16 + lr;
  const bool row_ok = row < a.d_out;
  const int64_t T = a.T, d = a.d;
  const int G = a.G;
  const int Tp = NTB * 16;
  const int64_t srow = (row_ok ? row : 0) * G;

  // the workgroup's rows of codes as one bounded buffer (rows past d_out and
  // groups past the end read as zeros, with no memory traffic)
  const int64_t rows_here = min((int64_t)16, a.d_out - rb * 16);
  const __amdgpu_buffer_rsrc_t cr =
      make_rsrc(a.packed + rb * 16 * a.row_bytes, (uint32_t)(rows_here * a.row_bytes));
  // lane quarter qd owns channels qd*GS/4 .. +GS/4 of each group
  const uint32_t lane_off =
      (uint32_t)(lr * a.row_bytes + qd * GroupCodes<CB, GS>::NB);

  auto load_g = [&](GroupCodes<CB, GS>& cv, int g) {
    const uint32_t soff = g < G ? (uint32_t)((int64_t)g * GS * CB / 8) : kOutOfRange;
    load_codes<CB, GS>(cv, cr, lane_off, soff);
  };

  f32x4 acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // T <= 16: the group's x' (fp16, scaled by a power of two per group and
  // token), its group sums and inverse scales, fetched with its codes one
  // group ahead (a group past the end fetches the last one again)
  struct XHL {
    u32x4 h[NKS];
    f32x4 sx, sc;
  };
  auto load_x = [&](XHL& x, int g) {
    if (!XF16) return;
    const int gg = g < G ? g : G - 1;
#pragma unroll
    for (int k = 0; k < NKS; ++k)
      x.h[k] = *(const u32x4*)(a.xs + 8 * xs_frag_index(gg, 0, k, l, 1, GS));
    x.sx = *(const f32x4*)(a.sx + (int64_t)gg * Tp + qd * 4);
    x.sc = *(const f32x4*)(a.xsc + (int64_t)gg * Tp + qd * 4);
  };

  auto process = [&](const GroupCodes<CB, GS>& cv, const XHL& x, int g) {
    const float s = a.s[srow + g];
    const float mb = a.m[srow + g] - BIAS * s;
    u32x4 qv[NKS];
#pragma unroll
    for (int k = 0; k < NKS; ++k) qv[k] = codes_operand<CB, F8, XF16>(step_codes<CB, GS>(cv, k));
    if (XF16) {
      f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NKS; ++k)
        P = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x.h[k]),
                                                  __builtin_bit_cast(f16x8, qv[k]), P, 0, 0, 0);
      // undo the token's power-of-two scale (exact), then s P + (m - BIAS s) sum(x')
      const f32x4 sxv = x.sx, scv = x.sc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[0][i] = fmaf(s, P[i] * scv[i], fmaf(mb, sxv[i], acc[0][i]));
    } else {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        u32x4 xv[NKS];
#pragma unroll
        for (int k = 0; k < NKS; ++k)
          xv[k] = *(const u32x4*)(a.xs + 8 * xs_frag_index(g, tb, k, l, NTB, GS));
        const f32x4 sxv = *(const f32x4*)(a.sx + (int64_t)g * Tp + tb * 16 + qd * 4);
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < NKS; ++k)
          P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, xv[k]), __builtin_bit_cast(bf16x8, qv[k]), P, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tb][i] = fmaf(s, P[i], fmaf(mb, sxv[i], acc[tb][i]));
      }
    }
  };

  // two register sets in ping-pong (a code request past the last group
  // reads nothing)
  GroupCodes<CB, GS> ca, cb;
  XHL xa, xb;
  int g = w;
  load_g(ca, g);
  load_x(xa, g);
  while (g < G) {
    load_g(cb, g + QF_W);
    load_x(xb, g + QF_W);
    __builtin_amdgcn_sched_barrier(0);
    process(ca, xa, g);
    g += QF_W;
    if (g >= G) break;
    load_g(ca, g + QF_W);
    load_x(xa, g + QF_W);
    __builtin_amdgcn_sched_barrier(0);
    process(cb, xb, g);
    g += QF_W;
  }

  // static low-rank term B (A X): one more MFMA chain on Z = A X
  if (a.rank > 0) {
    const int nk = a.rp / 32;
    for (int kk = w; kk < nk; kk += QF_W) {
      const int c8 = kk * 32 + qd * 8;
      const u32x4 bv = (row_ok && c8 < a.rank)
                           ? *(const u32x4*)(a.Blr + row * a.rank + c8)
                           : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const int64_t tok = tb * 16 + lr;
        const u32x4 zv = tok < T ? *(const u32x4*)(a.Z + tok * a.rp + c8)
                                 : u32x4{0u, 0u, 0u, 0u};
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, zv), __builtin_bit_cast(bf16x8, bv), acc[tb], 0, 0, 0);
      }
    }
  }

  // combine the waves in a fixed order; C of a 16x16 tile: lane l holds row
  // l & 15 and tokens 4 * (l >> 4) + i
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][tb * 4 + i][l] = acc[tb][i];
  __syncthreads();
  for (int e = tid; e < NTB * 256; e += QF_W * 64) {
    const int ti = e >> 6, ll = e & 63;
    const int64_t tok = (ti >> 2) * 16 + (ll >> 4) * 4 + (ti & 3);
    const int64_t rowx = rb * 16 + (ll & 15);
    if (tok < T && rowx < a.d_out) {
      float v = red[0][ti][ll];
#pragma unroll
      for (int ww = 1; ww < QF_W; ++ww) v += red[ww][ti][ll];
      a.Y[tok * a.d_out + rowx] = v;
    }
  }
}

template <int CB, int NTB, bool F8>
hipError_t launch_qf_ntb(const QFusedArgs& a, int group, dim3 grid,
                         const Launch& L) {
#define TTQ_QF_CASE(GSV)                                                     \
  case GSV:                                                                  \
    return ext_launch(k_qfused<CB, NTB, GSV, F8>, grid,                      \
                      dim3(qf_waves<NTB, GSV, F8>() * 64), 0, L, a);
  switch (group) {
    TTQ_QF_CASE(32)
    TTQ_QF_CASE(64)
    TTQ_QF_CASE(128)
    TTQ_QF_CASE(256)
    default: return hipErrorInvalidValue;
  }
#undef TTQ_QF_CASE
}

template <int CB, bool F8 = false>
hipError_t launch_qf_cb(const QFusedArgs& a, int ntb, int group, dim3 grid,
                        const Launch& L) {
  switch (ntb) {
    case 1: return launch_qf_ntb<CB, 1, F8>(a, group, grid, L);
    case 2: return launch_qf_ntb<CB, 2, F8>(a, group, grid, L);
    case 4: return launch_qf_ntb<CB, 4, F8>(a, group, grid, L);
    case 8: return launch_qf_ntb<CB, 8, F8>(a, group, grid, L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_qfused(const QFusedArgs& a, int ntb, int group, int cb,
                         const Launch& L) {
  const int64_t nblk = (a.d_out + 15) / 16;
  if (nblk == 0 || a.T == 0) return hipSuccess;
  if (a.T > 16 * ntb || (ntb == 1 && a.T > 16)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk);
  if (a.qf == QF_FP8)
    return cb == 8 ? launch_qf_cb<8, true>(a, ntb, group, grid, L) : hipErrorInvalidValue;
  switch (cb) {
    case 1: return launch_qf_cb<1>(a, ntb, group, grid, L);
    case 2: return launch_qf_cb<2>(a, ntb, group, grid, L);
    case 4: return launch_qf_cb<4>(a, ntb, group, grid, L);
    case 8: return launch_qf_cb<8>(a, ntb, group, grid, L);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ttq
