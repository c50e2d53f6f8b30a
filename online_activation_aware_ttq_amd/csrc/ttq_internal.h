// Internal declarations shared by the gfx950 kernels and the host layer of
// the TTQ linear projection.  Not part of the public ABI (include/ttq.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttq {

typedef uint16_t bf16_t;  // raw bfloat16 bit pattern
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// Kernel kinds, for the optional event timing.
enum KernelKind {
  K_STATS_SMALL = 0,   // norms + diag + scaled activations (T <= 128)
  K_STATS_Z,           // norms, partial sums per 64-token block (+ Z = X A^T)
  K_STATS_FINAL,       // norms finalize + diag
  K_FUSED,             // fused quantize + MFMA contraction (single W pass)
  K_QUANT,             // quantize pass writing W_hat (two-phase path)
  K_GEMM,              // MFMA GEMM Y = X W_hat^T + Z B^T (two-phase path)
  K_LOWRANK_Z,         // Z = X A^T (low-rank first factor)
  K_GEMV,              // single-launch path for one token (T = 1)
  K_SPLITK_REDUCE,     // split-K partial sums of Z -> bf16
  K_QGEMV,             // stored packed codes x one token
  K_DEQUANT,           // stored packed codes -> W_hat
  K_QFUSED,            // stored packed codes x 2..128 tokens
  K_LOWRANK_ZSUM,      // ordered sum of the small-M low-rank partials
  K_GEMM_Q,            // projection GEMM quantizing the weight tiles itself
  K_SEG_COPY,          // row copies for requests of different lengths
  K_SKINNY,            // PCA: skinny products with W and the panels
  K_PSUM,              // PCA: ordered sum of the split partials
  K_CHOL,              // PCA: Cholesky factor of a Gram matrix
  K_TRSM,              // PCA: panel times the inverse Cholesky factor
  K_LR_RESIDUAL,       // PCA: W - B A in bf16
  K_PCA_COMPLETE,      // PCA: completion of a rank-deficient basis
  K_STREAM_READ,       // plain read of device memory (measurement ceiling)
  K_NUM_KINDS
};

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float bf16lo(unsigned v) {
  return __uint_as_float(v << 16);
}
__device__ __forceinline__ float bf16hi(unsigned v) {
  return __uint_as_float(v & 0xffff0000u);
}
// float -> bfloat16 bits, round to nearest even (NaN stays NaN), with the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32).  Every kernel rounds
// through these two, so equal float32 values give equal bf16 bits on every
// path.
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  typedef __attribute__((ext_vector_type(2))) __bf16 b2;
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f2){lo, hi}, b2));
}
__device__ __forceinline__ unsigned f2bf(float f) {
  return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)f);
}

// Raw buffer loads: a resource descriptor bounds the addressable range, and a
// 16-byte load whose offset falls outside it returns zeros without touching
// memory.  Used to stream weight tiles with no branches for ragged edges.
// (Descriptor word 3 for the gfx9 family, which includes gfx950.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r,
                                            uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Same, non-temporal (streamed data that should not displace reused lines
// from the caches; cache-policy bit NT of the gfx94x/gfx950 encoding).
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r,
                                               uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
// Wait until every vector memory access of this wave has completed (gfx9
// s_waitcnt encoding: vmcnt[3:0] = 0, expcnt[6:4] = 7, lgkmcnt[11:8] = 15).
// Used to order a small dependent read ahead of a large batch of loads.
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Workgroup barrier for kernels that fill LDS with buffer_load ... lds:
// this wave's LDS accesses are complete (lgkmcnt 0), then s_barrier.  The
// direct-to-LDS loads are waited for explicitly through vmcnt, stage by
// stage; __syncthreads() would also wait for every such load in flight
// (vmcnt 0), which leaves a multi-stage load pipeline one stage deep.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// scalar offset that puts a load out of range (no wrap-around: the lane
// offsets of a weight tile stay far below 2^30)
constexpr uint32_t kOutOfRange = 0x40000000u;

// ---------------------------------------------------------------- formats
// Quantizer formats Q (the method leaves the code format open: the
// lo0 blog "Test-time quantization: quantising on the fly with no
// calibration dataset", section "What TTQ is NOT", calls it orthogonal to
// INT4 or FP8 codes).  For a group of u = w D^{1/2} with minimum mn and
// maximum mx every format decides a level L per element in float32 and
// reconstructs u_hat = s L + c:
//   QF_ASYM   s = (mx - mn) / N, c = mn, L = rint((u - mn) inv) in [0, N],
//             code L                                  (the default)
//   QF_SYM    s = max(-mn, mx) / Z, Z = 2^{b-1} - 1, c = 0,
//             L = clamp(rint(u inv), -Z, Z), code L + Z
//   QF_INTZP  lo = min(mn, 0), hi = max(mx, 0), s = (hi - lo) / N, c = 0,
//             z = rint(lo inv), L = clamp(rint(u inv), z, z + N), code L - z
//             (the affine form with an integer zero point: zero is exact)
//   QF_FP8    s = max(-mn, mx) / 448, c = 0, L = E4M3 rounding of
//             clamp(u inv, -448, 448) (nearest, ties to even), code = the
//             E4M3 bit pattern (OCP FP8, bias 7, no infinities; the sign
//             bit is that of u inv, also when L is zero)
// with inv = 1/s (0 when s = 0) and no fused operations.  Every level is
// exact in bf16 (integers of at most 9 bits, or 4 significant bits), so it
// can be an MFMA operand.  Beside the scales the library stores a per-group
// offset `off` with u_hat = off + s code for the integer formats (QF_SYM:
// -(Z s), QF_INTZP: z s; both one float32 rounding away from the exact
// reconstruction); it is 0 for QF_FP8, whose codes decode to E4M3 values.
enum QFmt : int { QF_ASYM = 0, QF_SYM = 1, QF_INTZP = 2, QF_FP8 = 3 };

struct QGroup {
  float s, inv;
  float c;       // subtracted before the scaling, added back in u_hat
  float lo, hi;  // level range
  float off;     // stored offset
};

// the group scale s of a format
template <int QF>
__device__ __forceinline__ float qscale(float mn, float mx, float Nf) {
  if constexpr (QF == QF_ASYM) return (mx - mn) / Nf;
  else if constexpr (QF == QF_INTZP) return (fmaxf(mx, 0.f) - fminf(mn, 0.f)) / Nf;
  else if constexpr (QF == QF_SYM) return fmaxf(-mn, mx) / ((Nf - 1.f) * 0.5f);
  else return fmaxf(-mn, mx) / 448.f;
}

// the rest of the group's constants, given s and inv = 1/s (0 if s = 0)
template <int QF>
__device__ __forceinline__ QGroup qgroup_si(float mn, float s, float inv,
                                            float Nf) {
  QGroup g;
  g.s = s;
  g.inv = inv;
  g.c = QF == QF_ASYM ? mn : 0.f;
  if constexpr (QF == QF_ASYM) {
    g.lo = 0.f;
    g.hi = Nf;
    g.off = mn;
  } else if constexpr (QF == QF_INTZP) {
    g.lo = __builtin_rintf(fminf(mn, 0.f) * inv);
    g.hi = g.lo + Nf;
    g.off = g.lo * s;
  } else if constexpr (QF == QF_SYM) {
    g.hi = (Nf - 1.f) * 0.5f;
    g.lo = -g.hi;
    g.off = -(g.hi * s);
  } else {
    g.lo = -448.f;
    g.hi = 448.f;
    g.off = 0.f;
  }
  return g;
}

template <int QF>
__device__ __forceinline__ QGroup qgroup(float mn, float mx, float Nf) {
  const float s = qscale<QF>(mn, mx, Nf);
  return qgroup_si<QF>(mn, s, s > 0.f ? 1.0f / s : 0.f, Nf);
}

// E4M3 on the gfx950 conversion unit: v_cvt_pk_fp8_f32 rounds to the
// nearest E4M3 value (ties to even, the sign kept, also for a zero result)
// and writes its bit pattern; v_cvt_f32_fp8 decodes a pattern.  On |t| <=
// 448 they agree bit for bit with the E4M3 definition (checked on MI355X over
// every float32 input of that range and every code).
__device__ __forceinline__ unsigned e4m3_code(float t) {
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(t, t, 0, false) & 0xffu;
}
__device__ __forceinline__ float e4m3_value(unsigned c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}
// value of byte b (0..3, a compile-time constant after unrolling) of w
__device__ __forceinline__ float e4m3_byte(unsigned w, int b) {
  switch (b & 3) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

template <int QF>
__device__ __forceinline__ float qlevel(const QGroup& g, float u) {
  if constexpr (QF == QF_ASYM)
    return __builtin_amdgcn_fmed3f(__builtin_rintf((u - g.c) * g.inv), 0.f, g.hi);
  else if constexpr (QF == QF_FP8)
    return e4m3_value(e4m3_code(__builtin_amdgcn_fmed3f(u * g.inv, g.lo, g.hi)));
  else
    return __builtin_amdgcn_fmed3f(__builtin_rintf(u * g.inv), g.lo, g.hi);
}

// levels of 8 elements; QF_FP8 converts pairs (one instruction each way per
// two elements)
template <int QF>
__device__ __forceinline__ void qlevels8(const QGroup& g, const float (&u)[8],
                                         float (&L)[8]) {
  if constexpr (QF == QF_FP8) {
    typedef __attribute__((ext_vector_type(2))) float f2;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int c = __builtin_amdgcn_cvt_pk_fp8_f32(
          __builtin_amdgcn_fmed3f(u[j] * g.inv, g.lo, g.hi),
          __builtin_amdgcn_fmed3f(u[j + 1] * g.inv, g.lo, g.hi), 0, false);
      const f2 v = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
      L[j] = v.x;
      L[j + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) L[j] = qlevel<QF>(g, u[j]);
  }
}

template <int QF>
__device__ __forceinline__ unsigned qcode(const QGroup& g, float L) {
  if constexpr (QF == QF_SYM) return (unsigned)(L + g.hi);
  else if constexpr (QF == QF_INTZP) return (unsigned)(L - g.lo);
  else if constexpr (QF == QF_FP8) return e4m3_code(L);
  else return (unsigned)L;
}


// Scaled activations x' = x D^{-1/2} as the fused kernels' MFMA operand, in
// MFMA fragment order over Tp = 16 * ceil(T / 16) tokens (zeros past T): the
// 16-byte fragment of lane l for group g, 16-token block tb and MFMA step k
// (k < GS / 32) holds tokens tb*16 + (l & 15) and 8 channels from
//   step-major order:  g*GS + 32k + 8*(l >> 4)        (the one-pass kernel:
//                      each wave load of weights covers 64 contiguous bytes
//                      of each of 16 rows), or
//   quarter order:     g*GS + (l >> 4) * GS/4 + 8k    (the packed-code kernel:
//                      a lane's codes of one group are one contiguous run),
// at fragment index ((g * NTB + tb) * (GS / 32) + k) * 64 + l, so that one
// wave load of a fragment is 1 KiB contiguous.
// One plane of Tp * d values: fp16 scaled per (group, token) for T <= 16,
// bf16 above.
__host__ __device__ inline int64_t xs_frag_index(int64_t g, int64_t tb,
                                                 int64_t k, int l, int ntb,
                                                 int gs) {
  return ((g * ntb + tb) * (gs / 32) + k) * 64 + l;
}

// ---------------------------------------------------------------- launchers
// Where and how to launch: the stream, plus optional events that the runtime
// stamps with the kernel's own start and end (measurement only).
struct Launch {
  hipStream_t s;
  hipEvent_t e0, e1;
};

template <typename... A>
inline hipError_t ext_launch(void (*kernel)(A...), dim3 grid, dim3 block,
                             uint32_t lds, const Launch& L, const A&... args) {
  void* argv[] = {const_cast<A*>(&args)...};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                            argv, lds, L.s, L.e0, L.e1, 0);
}

struct StatsSmallArgs {
  const bf16_t* X;      // [R][T][d]
  int64_t T, d;
  int pmode;            // 1: p == 1, 2: p == 2, 0: general p
  double p, lam, alpha;
  float* dh;            // [R][d]
  float* dhi;           // [R][d]
  float* dh_export;     // optional [R][d]
  bf16_t* xs;           // optional x * D^{-1/2} in bf16, see xs_frag_index
  float* sx;            // with xs: [R][G][Tp] group sums of xs, zero past T
  int group;
  int Tp;               // 16 * ceil(T / 16): tokens of the fragment layout
  int quarter;          // 1: quarter order of the fragments, 0: step-major
  // optional [R][d] stored D^{-1/2}: no statistics are taken, x' and the
  // group sums are formed with these values (dh, dhi are not written)
  const float* dhi_in;
  // optional (with xs): the float32 partials of Z = X A^T over each
  // 128-channel slice, [ceil(d / 128)][R * T][zrp], in the layout of the
  // small-M low-rank kernel's partials (its sum kernel finishes Z)
  const bf16_t* zA;     // [zrank][d]
  int zrank, zrp;
  float* zpart;
  // optional (with xs): x' as fp16 scaled by a power of two per (group,
  // token) instead of bf16, the inverse factors [R][G][Tp] here
  float* xsc;
};
hipError_t launch_stats_small(const StatsSmallArgs& a, int R,
                              const Launch& L);

// Large T (two-phase paths, quantize-once and PCA statistics): one pass over
// X per 64-token block that writes float64 partial powers per channel and,
// when asked for, the low-rank product Z = X A^T of the block's tokens.
struct StatsZArgs {
  const bf16_t* X;      // [R][T][d]
  int64_t T, d;
  int pmode;            // 1: p == 1, 2: p == 2, 0: general p
  double p;
  int ntb;              // 64-token blocks per request (ceil(T / 64))
  int csplit, cps;      // channel ranges per block, 512-channel chunks each
  double* partial;      // [R][ntb][d] sums of |x|^p over each block's tokens
  const bf16_t* A;      // [rank][d], or null: statistics only
  int rank, rp;         // rp = rank rounded up to 32, at most 128
  bf16_t* Z;            // csplit == 1: [R*T][rp] (columns past rank zero)
  float* Zpart;         // csplit > 1: [csplit][R*T][rp] fp32 partials
  int64_t zslice;       // R*T*rp: the stride of one channel range's partials
};
hipError_t launch_stats_z(const StatsZArgs& a, int R, const Launch& L);
size_t stats_z_lds_bytes();

// D^{+-1/2} from the block partials: nb partial rows per request, summed in
// order, then the norm, lambda and the power.
struct StatsFinalArgs {
  const double* partial;  // [R][nb][d]
  int64_t d;
  int nb;
  int pmode;
  double p, lam, alpha;
  float* dh;
  float* dhi;
  float* dh_export;
  // optional (zpart non-null): Z[i] = bf16(sum_{k<zsplit} zpart[k*zn + i])
  // in range order, i < zn (zn % 4 == 0), by extra workgroups of the launch
  const float* zpart;
  int zsplit;
  int64_t zn;
  bf16_t* Z;
  int R;                  // requests (set by the launcher)
};
hipError_t launch_stats_final(const StatsFinalArgs& a, int R, const Launch& L);

struct FusedArgs {
  const bf16_t* W;      // [d_out][d]
  int64_t d, d_out, T;
  int G;                // groups per row
  float Nf;             // 2^bits - 1
  const float* dh;      // [R][d]
  const bf16_t* xs;     // x * D^{-1/2}, layout as written by the stats kernel
  const float* sx;      // [R][G][Tp] group sums of xs, Tp = 16 * ntb,
                        // zero past T
  const float* xsc;     // ntb == 1: [R][G][Tp] inverse fp16 scales of xs
  const bf16_t* Z;      // [R][T][rp] or null
  const bf16_t* Blr;    // [d_out][rank] or null
  int rank, rp;
  float* Y;             // [R][T][d_out]
  int64_t rowblocks;    // ceil(d_out / 16)
  int R;
  uint8_t* codes_out;   // [R][d_out][d]
  float* s_out;         // [R][d_out][G]
  float* m_out;         // [R][d_out][G]
  int qf;               // quantizer format (QFmt)
};
// D^{1/2} is staged in LDS when it fits in this many bytes.
constexpr size_t kFusedDhLdsMax = 64 * 1024;
// rb: 16-row blocks per workgroup (1, or 2 for groups of up to 128 and
// ntb >= 2)
hipError_t launch_fused(const FusedArgs& a, int ntb, int group, int rb,
                        const Launch& L);

struct GemvArgs {
  const bf16_t* W;      // [d_out][d]
  const bf16_t* X;      // [R][d]   (one token per request)
  int64_t d, d_out;
  int G;
  float Nf;
  int pmode;
  double p, lam, alpha;
  const bf16_t* Z;      // [R][rp] or null
  const bf16_t* Blr;    // [d_out][rank] or null
  int rank, rp;
  float* Y;             // [R][d_out]
  int64_t rowblocks;
  int R;
  uint8_t* codes_out;   // [R][d_out][d]
  float* s_out;         // [R][d_out][G]
  float* m_out;
  float* dh_export;     // [R][d]
  int qf;               // quantizer format (QFmt)
};
// the single-launch T = 1 kernel holds all of D^{1/2} and x' in LDS
constexpr int64_t kGemvMaxD = 12288;
size_t gemv_lds_bytes(int64_t d, int G);
hipError_t launch_gemv(const GemvArgs& a, int group, const Launch& L);

struct QuantArgs {
  const bf16_t* W;      // [d_out][d], shared by the requests
  int64_t d, d_out;
  int G;
  int R;                // requests, each with its own statistics
  float Nf;
  const float* dh;      // [R][d]
  const float* dhi;     // [R][d]
  bf16_t* What;         // [R][what_tiled_elems(d_out, d)], tiled (see below)
  uint8_t* codes_out;   // [R][d_out][d]
  float* s_out;         // [R][d_out][G]
  float* m_out;         // [R][d_out][G]
  // packed-code output instead of W_hat (What unused when set)
  uint8_t* packed;      // [R][d_out][row_bytes]
  int cb;               // container bits 1, 2, 4, 8
  int64_t row_bytes;    // d * cb / 8
  int qf;               // quantizer format (QFmt)
};
hipError_t launch_quant(const QuantArgs& a, int group, const Launch& L);

// Contraction of later tokens with stored packed codes (one token):
// y_i = sum_g s_ig * sum_{j in g} q_ij x'_j + m_ig * sum_{j in g} x'_j
// + B_i . z, with x' = x D^{-1/2} from the stored D^{-1/2}.
struct QGemvArgs {
  const uint8_t* packed;  // [d_out][row_bytes]
  int64_t row_bytes;
  const float* s;         // [d_out][G]
  const float* m;         // [d_out][G]
  const float* dhi;       // [d]
  const bf16_t* X;        // [d] (one token)
  int64_t d, d_out;
  int G;
  const bf16_t* Z;        // [rp] or null
  const bf16_t* Blr;      // [d_out][rank] or null
  int rank;
  float* Y;               // [d_out]
  int qf;                 // QF_FP8: E4M3 codes; any other format: integer codes
};
hipError_t launch_qgemv(const QGemvArgs& a, int group, int cb, const Launch& L);
size_t qgemv_lds_bytes(int64_t d, int cb, int group);

// Dequantize stored packed codes to W_hat = bf16((m + s q) D^{-1/2}).
struct DequantArgs {
  const uint8_t* packed;  // [d_out][row_bytes]
  int64_t row_bytes;
  const float* s;
  const float* m;
  const float* dhi;
  int64_t d, d_out;
  int G;
  bf16_t* What;           // [d_out][d]
  int qf;                 // QF_FP8: E4M3 codes; any other format: integer codes
};
hipError_t launch_dequant(const DequantArgs& a, int group, int cb,
                          const Launch& L);

// Contraction of 2..128 later tokens with stored packed codes on the matrix
// cores (same x' operand and group sums as the fused one-pass kernel, written
// by the statistics kernel from the stored D^{-1/2}).
struct QFusedArgs {
  const uint8_t* packed;  // [d_out][row_bytes]
  int64_t row_bytes;
  const float* s;         // [d_out][G]
  const float* m;         // [d_out][G]
  const bf16_t* xs;       // x' as written by the statistics kernel
  const float* sx;        // [G][Tp] group sums of xs
  const float* xsc;       // T <= 16: [G][16] inverse fp16 scales of xs
  int64_t d, d_out, T;
  int G;
  const bf16_t* Z;        // [T][rp] or null
  const bf16_t* Blr;      // [d_out][rank] or null
  int rank, rp;
  float* Y;               // [T][d_out]
  int qf;                 // QF_FP8: E4M3 codes; any other format: integer codes
};
hipError_t launch_qfused(const QFusedArgs& a, int ntb, int group, int cb,
                         const Launch& L);

// Layout of the W_hat the quantize pass writes for the GEMM: tiles of 256
// rows x 64 channels stored contiguously (32 KiB), the tiles of a 256-row
// block in channel order, blocks in row order:
//   element (n, k) at ((n / 256) * ceil(K / 64) + k / 64) * 16384
//                     + (n % 256) * 64 + k % 64.
// One direct-to-LDS load of the GEMM (8 rows x 64 channels) is then 1 KiB of
// contiguous memory instead of 8 row pieces 2 d bytes apart (measured on the
// 7B-class layer: 5-14 % less GEMM time than row-major rows padded to
// d + 64, which were themselves 6-11 % faster than unpadded rows).  Rows
// past d_out in the last block are never written; the GEMM reads them only
// into output columns it does not store.  Channels past K are not read.
constexpr int64_t kWtRows = 256, kWtCols = 64;
__host__ __device__ inline int64_t what_tiled_elems(int64_t d_out, int64_t K) {
  return (d_out + kWtRows - 1) / kWtRows * kWtRows * ((K + kWtCols - 1) / kWtCols) * kWtCols;
}
__host__ __device__ inline int64_t what_tiled_index(int64_t n, int64_t k, int64_t nk) {
  return ((n / kWtRows) * nk + k / kWtCols) * (kWtRows * kWtCols) + (n % kWtRows) * kWtCols +
         k % kWtCols;
}

// C[M][N] (+)= A1[M][K1] B1[N][K1]^T + A2[M][K2] B2[N][K2]^T, fp32 accumulate.
struct GemmArgs {
  const bf16_t* A1; int64_t lda1;
  const bf16_t* B1; int64_t ldb1;
  int64_t K1;
  int b1_tiled;                     // B1 in the tiled W_hat layout (ldb1 unused)
  const bf16_t* A2; int64_t lda2;   // optional second segment (low rank)
  const bf16_t* B2; int64_t ldb2;
  int64_t K2;
  int64_t M, N;
  int64_t N_store;                  // columns actually stored (<= ldc)
  float* C; int64_t ldc;            // fp32 output, or
  bf16_t* Cb;                       // bf16 output (one of the two)
  // split-K (first segment only, fp32 output): split z covers channels
  // [z*ksplit, (z+1)*ksplit) and writes C + z*split_stride
  int64_t ksplit;                   // multiple of 64; 0 = no split
  int nsplit;
  int64_t split_stride;
  // batch of independent products (large-tile kernel): product z uses
  // A1 + z*sA1, B1 + z*sB1, A2 + z*sA2, B2 + z*sB2 and writes C + z*sC
  int batch;                        // 0 or 1 = a single product
  int64_t sA1, sB1, sA2, sB2, sC;
};
hipError_t launch_gemm(const GemmArgs& a, const Launch& L);
// Large-tile variant for the projection GEMM (fp32 C, no split): operands
// streamed into LDS by direct loads.  gemm_lds_config: 0 = 256 x 256 tiles,
// persistent workgroups, 1 = 256 x 128 tiles, 2 = 256 x 256 tiles, one per
// workgroup.
hipError_t launch_gemm_lds(const GemmArgs& a, const Launch& L);
int gemm_lds_config(int64_t M, int64_t N, int64_t batch);

// Projection GEMM with the weight operand quantized in the kernel:
//   C[M][N] = X[M][K1] * W_hat[N][K1]^T  +  A2[M][K2] * B2[N][K2]^T
// where W_hat = bf16((m + s q) D^{-1/2}) is formed from the bf16 weights W and
// the product's D^{+-1/2} tile by tile, with the same float32 decisions as
// the quantize pass (the results are identical to quantize pass + GEMM).
// Products of a batch share W and have their own X, D^{+-1/2}, A2 and C.
// With stored codes instead of W (cb > 0), W_hat = bf16((m + s q) D^{-1/2})
// from the codes' CB-bit containers and the per-group s, m (one product).
struct GemmQArgs {
  const bf16_t* X; int64_t ldx;
  const bf16_t* W; int64_t ldw;
  const uint8_t* packed; int64_t row_bytes;   // codes (cb > 0)
  const float* s; const float* m; int64_t G;  // [N][G] (cb > 0)
  const float* dh;      // [batch][K1] (cb = 0)
  const float* dhi;     // [batch][K1]
  float Nf;             // 2^bits - 1
  int64_t K1;
  const bf16_t* A2; int64_t lda2;   // optional low-rank segment
  const bf16_t* B2; int64_t ldb2;
  int64_t K2;
  int64_t M, N;
  float* C; int64_t ldc;
  int batch;
  int64_t sX, sA2, sC;  // per-product strides (elements); D^{+-1/2}: K1
  int qf;               // quantizer format (QFmt); with codes: QF_FP8 decodes
                        // E4M3 codes, every other value integer codes
};
hipError_t launch_gemm_q(const GemmQArgs& a, int group, int cb, const Launch& L);
// K1 a multiple of 128; groups of 32, 64 or 128 channels (also 256 when
// expanding codes, cb > 0)
bool gemm_q_supported(int64_t K1, int group, int cb);

// Row copies between a packed multi-request array and a padded batch (see
// k_segment.hip).  Rows are row_bytes long (a multiple of 4).
constexpr int kSegMax = 64;  // requests per copy launch
struct SegCopyArgs {
  const void* src;
  void* dst;
  int64_t row_bytes;
  int64_t Tpad;             // rows per request in the padded batch
  int n;                    // requests in this launch
  int scatter;              // 0: packed -> padded (zero fill), 1: padded -> packed
  int64_t off[kSegMax];     // first row of request r in the packed array
  int64_t len[kSegMax];     // rows of request r
};
hipError_t launch_seg_copy(const SegCopyArgs& a, const Launch& L);

// ---- low-rank factors by PCA (k_pca.hip)
// one skinny product C[rows][n] = A_s Bm (A read row-wise: A[row][k]) or
// A_s^T Bm (A read column-wise: A[k][row]), over K, as split-K partials
// part[split][rows][n]; A is bf16 or float32, its columns (the index along a
// memory row) optionally scaled by `scale`
struct SkinnyArgs {
  const void* A; int64_t lda;
  const float* scale;     // optional, per column of A in memory
  const float* Bm; int64_t ldb;   // [K][ldb] float32
  int64_t rows, K;
  int n;                  // 8, 16, 32, 64 or 128
  int64_t kc;             // channels per split, a multiple of 64
  float* part;            // [ceil(K / kc)][rows][n]
};
hipError_t launch_skinny(const SkinnyArgs& a, bool tn, bool a_bf16, const Launch& L);
int skinny_splits(int64_t rows, int64_t K);
int64_t skinny_kc(int64_t K, int splits);
// out = sum of the nsplit partials in order (float32 [rows][n]), optionally
// also as bf16 [rows][n] and / or bf16 transposed [n][rows]
struct PsumArgs {
  const float* part;
  int nsplit;
  int64_t rows, n;
  float* out;
  bf16_t* out_bf16;
  bf16_t* out_bf16_t;
};
hipError_t launch_psum(const PsumArgs& a, const Launch& L);
// Cholesky factor R (upper, G = R^T R) of an n x n Gram matrix (n <= 128),
// and Y[m][n] <- Y R^{-1} in place
// (defic, optional: n flags, 1 where the pivot was raised to the floor)
hipError_t launch_chol(const float* G, float* R, int n, int* defic,
                       const Launch& L);
hipError_t launch_trsm(float* Y, const float* R, int64_t m, int n, const Launch& L);
// n <= 64: R^{-1} of the Cholesky factor in one wave (float64 registers)
hipError_t launch_cholinv(const float* G, float* Rinv, int n, int* defic,
                          const Launch& L);
// flagged columns of V [m][n] <- pseudo-random +-1/sqrt(m) columns (n <= 128)
hipError_t launch_pca_complete(float* V, int64_t m, int n, const int* defic,
                               const Launch& L);
struct LrResidualArgs {
  const bf16_t* W;        // [d_out][d]
  const bf16_t* B;        // [d_out][n]
  const bf16_t* A;        // [n][d]
  bf16_t* Wres;           // [d_out][d]
  int64_t d, d_out;
};
hipError_t launch_lr_residual(const LrResidualArgs& a, int n, const Launch& L);

// out[i] = bf16(sum_{z<nsplit} part[z*n + i]) in split order, n % 4 == 0
struct SplitReduceArgs {
  const float* part;
  int nsplit;
  int64_t n;
  bf16_t* out;
};
hipError_t launch_splitk_reduce(const SplitReduceArgs& a, const Launch& L);

struct LowRankZArgs {
  const bf16_t* X;      // [M][d]
  const bf16_t* A;      // [rank][d]
  int64_t M, d;
  int rank, rp;
  bf16_t* Z;            // [M][rp]
  float* part;          // [nsplit][M][rp] fp32 partial sums (workspace)
};
// Z = X A^T for small M: channel slices on the matrix cores (partials), then
// their sum in slice order.  Two launches; lowrank_z_splits gives the slice
// count and lowrank_z_part_bytes the bytes of `part` (256-channel slices;
// 128 where the small-T statistics kernel writes the partials).
hipError_t launch_lowrank_z_small(const LowRankZArgs& a, const Launch& L);
hipError_t launch_lowrank_z_sum(const LowRankZArgs& a, int nsplit, const Launch& L);
int lowrank_z_splits(int64_t M, int64_t d, int rp, int slice);
inline size_t lowrank_z_part_bytes(int64_t M, int64_t d, int rp, int slice) {
  return (size_t)lowrank_z_splits(M, d, rp, slice) * M * rp * sizeof(float);
}

// Plain streaming read (measurement ceiling of the one-token projection):
// one workgroup per kStreamReadBlockBytes, one XOR per workgroup to sink.
constexpr int64_t kStreamReadBlockBytes = 128 * 1024;
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                              const Launch& L);

}  // namespace ttq
