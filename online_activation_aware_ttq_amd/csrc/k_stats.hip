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
// For T <= 16 one outlier channel can dominate every output of a token, and
// a single bf16 rounding of its x' would be shared by all of them: x' is
// written in fp16 (11 significant bits) scaled by a power of two per (group,
// token) so that any float32 magnitude fits, with the inverse factors in
// their own array.  For larger T x' is written in bf16.  The plane is in
// MFMA fragment order (xs_frag_index) and zero-padded to whole 16-token
// blocks.  The group sums are of exactly the
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

  // Bounded buffer loads over the request's rows: tokens past T and chunks
  // past d read zeros with no branch, so all NTK loads are in flight at
  // once (guarded loads were waited for in pairs, one round trip each).
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)(a.T * a.d * 2));
  u32x4 v[NTK];
#pragma unroll
  for (int i = 0; i < NTK; ++i) {
    const int64_t t = tl + i * TLN;
    const uint32_t off = live ? (uint32_t)((t * a.d + c0) * 2) : kOutOfRange;
    v[i] = buf_load16(xr, off, 0);
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

  const int ntb = a.Tp / 16;
  const int G = (int)(a.d / a.group);
  const int lpg = a.group >> 3;  // chunk lanes per quantization group
  bf16_t* xs = a.xs + (int64_t)r * a.Tp * a.d;
  float* sx = a.sx + (int64_t)r * G * a.Tp;
  // scaled fp16 form (one plane): x' of a (group, token) is stored as
  // fp16(x' 2^k), k chosen from the group's largest |x'| so that it lands in
  // [2^14, 2^15); 2^-k goes to xsc.  The power of two is exact, so only the
  // fp16 rounding remains (11 significant bits) at any float32 magnitude.
  const bool f16s = a.xsc != nullptr;
  float* xsc = f16s ? a.xsc + (int64_t)r * G * a.Tp : nullptr;
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
    u32x4 o = {0u, 0u, 0u, 0u};
    const bool have = live && t < a.T;
    const float x[8] = {bf16lo(v[i].x), bf16hi(v[i].x), bf16lo(v[i].y),
                        bf16hi(v[i].y), bf16lo(v[i].z), bf16hi(v[i].z),
                        bf16lo(v[i].w), bf16hi(v[i].w)};
    float inv_scale = 1.f;
    if (f16s) {  // uniform
      float xp[8], gm = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xp[j] = x[j] * sc[j];
        gm = fmaxf(gm, fabsf(xp[j]));
      }
      if (!have) gm = 0.f;
      // the group's largest |x'| over its adjacent chunk lanes
      for (int off = lpg >> 1; off > 0; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
      // gm in [2^(e-1), 2^e): scale by 2^k, k = 15 - e (at most 126)
      const int k = gm > 0.f ? min(126, 15 - __builtin_amdgcn_frexp_expf(gm)) : 0;
      const float scale = __builtin_amdgcn_ldexpf(1.f, k);
      inv_scale = __builtin_amdgcn_ldexpf(1.f, -k);
      if (have) {
        unsigned hb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const _Float16 h = (_Float16)(xp[j] * scale);
          hb[j] = (unsigned)__builtin_bit_cast(unsigned short, h);
          ps += (float)h * inv_scale;
        }
        o = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16),
                  hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
      }
    } else if (have) {
      unsigned bh[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bh[j] = f2bf(x[j] * sc[j]);
        ps += __uint_as_float(bh[j] << 16);
      }
      o = u32x4{bh[0] | (bh[1] << 16), bh[2] | (bh[3] << 16),
                bh[4] | (bh[5] << 16), bh[6] | (bh[7] << 16)};
    }
    if (live) {
      const int lane = lane_q + (int)(t & 15);
      const int64_t fi = 8 * xs_frag_index(g, t >> 4, k, lane, ntb, a.group);
      *(u32x4*)(xs + fi) = o;
    }
    // the chunk lanes of one group are adjacent within a token row
    for (int off = lpg >> 1; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    if (live && (cq % lpg) == 0) {
      sx[g * a.Tp + t] = ps;
      if (f16s) xsc[g * a.Tp + t] = inv_scale;
    }
  }

  // Low-rank partials of this workgroup's 128-channel slice(s) and 32
  // tokens (Z = X A^T, summed over the slices by k_lowrank_zsum): per 16
  // tokens x 16 rank columns, one v_mfma_f32_16x16x32_bf16 from zero for
  // each 32-channel quarter of the slice (zero-filled past d, T and the
  // rank), added in quarter order.  A token's partials depend only on its
  // row of X and on A.
  if (a.zpart) {
    constexpr int NSL = BC / 128;
    constexpr uint32_t kPastEnd = 0xFFFFFFF0u;   // past any row range below
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(a.zA, (uint32_t)((int64_t)a.zrank * a.d * 2));
    const int l = tid & 63, tr = l & 15, kq = l >> 4;
    const int ntr = a.zrp / 16;
    const int64_t M = (int64_t)gridDim.z * a.T;
    const int jobs = 2 * ntr * NSL;
    for (int j = wv; j < jobs; j += NWV) {
      const int tt = j & 1, rt = (j >> 1) % ntr, sl = (j >> 1) / ntr;
      const int64_t t0 = (int64_t)blockIdx.y * 32 + tt * 16;
      const int64_t zs = (int64_t)blockIdx.x * NSL + sl;
      if (t0 >= a.T || zs * 128 >= a.d) continue;  // uniform per wave
      const int64_t tk = t0 + tr;
      const int rrow = rt * 16 + tr;
      const bool tok = tk < a.T, rok = rrow < a.zrank;
      // bounded loads (zeros past d, T and the rank, no branch: all eight
      // in flight at once)
      u32x4 xf[4], af[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int64_t c = zs * 128 + 32 * qq + 8 * kq;
        const bool cin = c < a.d;
        xf[qq] = buf_load16(xr, cin && tok ? (uint32_t)((tk * a.d + c) * 2) : kPastEnd, 0);
        af[qq] = buf_load16(ar, cin && rok ? (uint32_t)(((int64_t)rrow * a.d + c) * 2) : kPastEnd, 0);
      }
      f32x4 q[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        q[qq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, xf[qq]), __builtin_bit_cast(bf16x8, af[qq]),
            f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 4 * (l >> 4) + i;
        if (t < a.T)
          a.zpart[(zs * M + (int64_t)r * a.T + t) * a.zrp + rt * 16 + (l & 15)] =
              ((q[0][i] + q[1][i]) + q[2][i]) + q[3][i];
      }
    }
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
// Large T: one workgroup (8 waves) per 64-token block of a request and range
// of channels.  X streams through LDS in chunks of 512 channels with
// buffer_load ... lds (two 64 KiB stages, the GEMM's swizzled 128-byte rows,
// channel block j of a chunk at j * 8 KiB), and every chunk is used twice:
//  * statistics: wave w owns the 64 channels of block w, lane (o, g) the
//    channels 8o .. 8o+7 of the tokens g, g+8, ..., g+56; float64 sums of
//    |x|^p over those tokens, then over the eight token groups (DPP, fixed
//    order), one float64 partial per channel and block;
//  * low rank (optional): wave w contracts its channel block with the same
//    channels of A on v_mfma_f32_32x32x16_bf16 (both 32-token halves of the
//    block, rank tiles of 32), accumulating over all chunks; the eight waves'
//    products are added in LDS in wave order and Z is rounded once to bf16
//    (or stored as a float32 partial of the channel range).
// So X is read once for both, and the token block's Z needs no partials
// when one range covers all channels.  The result depends on d, T and the
// channel ranges only: a request's statistics are the same in any batch.
// ---------------------------------------------------------------------------
namespace {

constexpr int kZTB = 64;                    // tokens per workgroup
constexpr int kZCW = 512;                   // channels per chunk
constexpr int kZStage = kZTB * kZCW * 2;    // 64 KiB

__device__ __forceinline__ int zswz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

template <int N>
__device__ __forceinline__ void zwait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)b, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

}  // namespace

// PM: p mode (2, 1, 0 = general p); RT: rank tiles of 32 (0 = statistics only)
template <int PM, int RT>
__global__ __launch_bounds__(512, 1) void k_stats_z(StatsZArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t b = blockIdx.x;
  const int split = (int)(b % a.csplit);
  b /= a.csplit;
  const int64_t tb = b % a.ntb, r = b / a.ntb;
  const int64_t t0 = tb * kZTB;
  const int64_t trows = min((int64_t)kZTB, a.T - t0);
  const int64_t cbeg = (int64_t)split * a.cps * kZCW;
  const int64_t cend = min(a.d, cbeg + (int64_t)a.cps * kZCW);
  const int nck = (int)((cend - cbeg + kZCW - 1) / kZCW);
  // rows past the block's tokens read as zeros (no traffic)
  const auto rx = make_rsrc(a.X + (r * a.T + t0) * a.d, (uint32_t)(trows * a.d * 2));

  // loads: wave w, instruction j fills rows 8w .. 8w+7 of channel block j;
  // lane l writes row 8w + l/8, physical chunk l%8 = logical (l%8)^zswz(row)
  const int lrow = w * 8 + (l >> 3);
  const int lch = (l & 7) ^ zswz(lrow);
  auto issue = [&](int kc, int stage) {
    const int64_t cb0 = cbeg + (int64_t)kc * kZCW;
    unsigned char* st = smem + stage * kZStage + w * 1024;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = cb0 + j * 64 + lch * 8;
      const uint32_t vo =
          (kc < nck && c < cend) ? (uint32_t)((lrow * a.d + c) * 2) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(st + j * 8192), 16, vo, 0, 0, 0);
    }
  };

  // statistics lanes: token group g, channel octet o of block w
  const int g = l & 7, o = l >> 3;
  // low-rank lanes: MFMA row l%32, 8-channel half l/32 of each 16-channel step
  const auto ra = make_rsrc(a.A, (uint32_t)((int64_t)a.rank * a.d * 2));
  constexpr int NZ = RT > 0 ? RT : 1;
  f32x16 zacc[2][NZ];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int rt = 0; rt < NZ; ++rt)
#pragma unroll
      for (int q = 0; q < 16; ++q) zacc[tt][rt][q] = 0.f;

  issue(0, 0);
  for (int kc = 0; kc < nck; ++kc) {
    const int stage = kc & 1;
    const int64_t cb0 = cbeg + (int64_t)kc * kZCW;
    // the rank rows' channels of this chunk (their latency hides behind the
    // statistics work); channels past the range meet zero activations
    u32x4 bfr[NZ][4];
    if constexpr (RT > 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int64_t c = cb0 + w * 64 + kk * 16 + (l >> 5) * 8;
          const int row = rt * 32 + (l & 31);
          const uint32_t vo = c < cend ? (uint32_t)((row * a.d + c) * 2) : kOutOfRange;
          bfr[rt][kk] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, vo, 0, 0));
        }
    }
    // the next chunk into the other stage (retired by the last barrier)
    issue(kc + 1, stage ^ 1);
    // this chunk landed (the rank loads and the next chunk may be in flight)
    zwait_vm<8 + 4 * RT>();
    lds_barrier();
    const unsigned char* st = smem + stage * kZStage + w * 8192;
    if constexpr (PM >= 0) {
      double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = i * 8 + g;
        const u32x4 v = *(const u32x4*)(st + row * 128 + ((o ^ zswz(row)) * 16));
        accum8(acc, v, PM, a.p);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[j] = acc[j] + dpp64<0xB1>(acc[j]);    // quad_perm [1,0,3,2]
        acc[j] = acc[j] + dpp64<0x4E>(acc[j]);    // quad_perm [2,3,0,1]
        acc[j] = acc[j] + dpp64<0x141>(acc[j]);   // row_half_mirror
      }
      const int64_t c = cb0 + w * 64 + o * 8;
      if (g == 0 && c < cend) {
        double* P = a.partial + (r * a.ntb + tb) * a.d + c;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          typedef __attribute__((ext_vector_type(2))) double d2;
          *(d2*)(P + j) = d2{acc[j], acc[j + 1]};
        }
      }
    }
    if constexpr (RT > 0) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 af[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int row = tt * 32 + (l & 31);
          const int ch = ((kk << 1) | (l >> 5)) ^ zswz(row);
          af[tt] = *(const u32x4*)(st + row * 128 + ch * 16);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            zacc[tt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, af[tt]), __builtin_bit_cast(bf16x8, bfr[rt][kk]),
                zacc[tt][rt], 0, 0, 0);
      }
    }
    lds_barrier();   // every wave is done with this stage
  }
  // the load issued past the last chunk still writes LDS
  zwait_vm<0>();
  lds_barrier();

  if constexpr (RT > 0) {
    // the eight waves' products, added in wave order
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        // C layout of a 32x32 tile: lane l holds column l%32 and rows
        // 8*(q/4) + 4*(l/32) + q%4
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = 8 * (q >> 2) + 4 * (l >> 5) + (q & 3);
          red[w * 1024 + m * 32 + (l & 31)] = zacc[tt][rt][q];
        }
        lds_barrier();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int oi = tid + h * 512;
          float v = red[oi];
#pragma unroll
          for (int ww = 1; ww < 8; ++ww) v += red[ww * 1024 + oi];
          const int64_t tok = t0 + tt * 32 + (oi >> 5);
          if (tok < a.T) {
            const int64_t zi = (r * a.T + tok) * a.rp + rt * 32 + (oi & 31);
            if (a.csplit == 1)
              a.Z[zi] = (bf16_t)f2bf(v);
            else
              a.Zpart[(int64_t)split * a.zslice + zi] = v;
          }
        }
        lds_barrier();
      }
  }
}

size_t stats_z_lds_bytes() { return 2 * (size_t)kZStage; }

namespace {
template <int PM, int RT>
hipError_t launch_sz(const StatsZArgs& a, unsigned nblk, const Launch& L) {
  constexpr uint32_t lds = 2 * kZStage;
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(k_stats_z<PM, RT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  return ext_launch(k_stats_z<PM, RT>, dim3(nblk), dim3(512), lds, L, a);
}
template <int PM>
hipError_t launch_sz_rt(const StatsZArgs& a, unsigned nblk, const Launch& L) {
  switch (a.A ? a.rp / 32 : 0) {
    case 0: return launch_sz<PM, 0>(a, nblk, L);
    case 1: return launch_sz<PM, 1>(a, nblk, L);
    case 2: return launch_sz<PM, 2>(a, nblk, L);
    case 3: return launch_sz<PM, 3>(a, nblk, L);
    case 4: return launch_sz<PM, 4>(a, nblk, L);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_stats_z(const StatsZArgs& a, int R, const Launch& L) {
  const int64_t nblk = (int64_t)R * a.ntb * a.csplit;
  if (nblk == 0) return hipSuccess;
  if (a.A && (a.rp % 32 != 0 || a.rp > 128 || a.rank > a.rp)) return hipErrorInvalidValue;
  if (a.d % 8 != 0 || (int64_t)kZTB * a.d * 2 >= (int64_t)kOutOfRange) return hipErrorInvalidValue;
  if (a.pmode == 2) return launch_sz_rt<2>(a, (unsigned)nblk, L);
  if (a.pmode == 1) return launch_sz_rt<1>(a, (unsigned)nblk, L);
  return launch_sz_rt<0>(a, (unsigned)nblk, L);
}

// One thread per channel; the block partials are read 8 at a time (independent
// loads in flight) and added in block order.
__global__ __launch_bounds__(64) void k_stats_final(StatsFinalArgs a) {
  if ((int)blockIdx.y >= a.R) {
    // the low-rank partial sum's workgroups (the split-K reduction of the
    // statistics pass's Z ranges): 4 consecutive elements per thread
    const int64_t i =
        (((int64_t)(blockIdx.y - a.R) * gridDim.x + blockIdx.x) * 64 + threadIdx.x) * 4;
    if (i >= a.zn) return;
    f32x4 acc = *(const f32x4*)(a.zpart + i);
    for (int z = 1; z < a.zsplit; ++z) {
      const f32x4 v = *(const f32x4*)(a.zpart + (int64_t)z * a.zn + i);
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    u32x2 o;
    o.x = pack_bf16(acc[0], acc[1]);
    o.y = pack_bf16(acc[2], acc[3]);
    *(u32x2*)(a.Z + i) = o;
    return;
  }
  const int r = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (c >= a.d) return;
  const int nb = a.nb;
  const double* P = a.partial + (int64_t)r * nb * a.d + c;
  // block order; the loads of 8 blocks are in flight together
  double S = 0.0;
  for (int k0 = 0; k0 < nb; k0 += 8) {
    double v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = k0 + j < nb ? P[(int64_t)(k0 + j) * a.d] : 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < nb) S += v[j];
  }
  float dh, dhi;
  diag_half(finish_norm(S, a.pmode, a.p), a.lam, a.alpha, dh, dhi);
  a.dh[(int64_t)r * a.d + c] = dh;
  a.dhi[(int64_t)r * a.d + c] = dhi;
  if (a.dh_export) a.dh_export[(int64_t)r * a.d + c] = dh;
}

hipError_t launch_stats_final(const StatsFinalArgs& a0, int R, const Launch& L) {
  StatsFinalArgs a = a0;
  a.R = R;
  const unsigned gx = (unsigned)((a.d + 63) / 64);
  unsigned zrows = 0;
  if (a.zpart && a.zn > 0) {
    if (a.zn % 4 != 0 || a.zsplit < 1 || !a.Z) return hipErrorInvalidValue;
    const int64_t wgs = (a.zn / 4 + 63) / 64;
    zrows = (unsigned)((wgs + gx - 1) / gx);
  }
  if ((R == 0 || a.d == 0) && zrows == 0) return hipSuccess;
  dim3 grid(gx > 0 ? gx : 1u, (unsigned)R + zrows);
  return ext_launch(k_stats_final, grid, dim3(64), 0, L, a);
}

}  // namespace ttq
