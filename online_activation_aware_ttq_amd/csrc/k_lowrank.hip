// First factor of the static low-rank term of TTQ for small token counts:
//   Z[m][k] = sum_j X[m][j] * A[k][j]       (Z = X A^T, i.e. (A X)^T)
// ("TTQ: Activation-Aware Test-Time Quantization ...", gist.science zh
// summary, Sec. 2.2: W ~ W_q + B A with static B, A).  Stored as bf16 with the
// rank padded to a multiple of 32 (zeros), the operand layout the fused
// kernels' MFMA tail reads.
//
// With few tokens the work is a long, thin reduction over the channels, so it
// is cut along the channels: a workgroup of 4 waves takes 16 tokens, 64 rank
// columns and one channel slice; each wave runs v_mfma_f32_16x16x32_bf16 over
// a quarter of the slice (A operand: 16 tokens x 32 channels of X, one 16-byte
// load per lane; B operand: 32 channels x 16 rank rows of A, likewise), the
// waves are added in LDS in a fixed order and the slice's fp32 partial tile
// is stored.  A second kernel adds the slices in slice order and rounds once
// to bf16, so the result does not depend on scheduling.  On the fused route
// (2 to 128 tokens) the small-T statistics kernel writes such partials
// itself, over 128-channel slices, and only the sum kernel runs.
#include "ttq_internal.h"

namespace ttq {

namespace {

constexpr int ZW = 4;        // waves per workgroup
constexpr int ZTILES = 4;    // 16-column rank tiles per workgroup

__global__ __launch_bounds__(ZW * 64) void k_lowrank_zpart(LowRankZArgs a,
                                                           int64_t kslice) {
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int n0 = blockIdx.y * 16 * ZTILES;
  const int z = blockIdx.z;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = min(ZTILES, (a.rp - n0) / 16);
  const int tr = l & 15, kq = l >> 4;
  const int64_t kbeg = (int64_t)z * kslice;
  const int64_t kend = min(a.d, kbeg + kslice);
  const int64_t wsl = kslice / ZW;
  const int64_t k0 = kbeg + w * wsl, k1 = min(kend, k0 + wsl);

  f32x4 acc[ZTILES];
#pragma unroll
  for (int t = 0; t < ZTILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operands of one 32-channel step (zero past the slice, past M, past
  // rank), as bounded buffer loads with no branch, so that the compiler
  // keeps both steps' loads in flight (guarded loads were waited for one by
  // one)
  constexpr uint32_t kPastEnd = 0xFFFFFFF0u;
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc(a.X + m0 * a.d, (uint32_t)(min((int64_t)16, a.M - m0) * a.d * 2));
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(a.A, (uint32_t)((int64_t)a.rank * a.d * 2));
  auto load = [&](int64_t kc, u32x4& xf, u32x4 (&af)[ZTILES]) {
    const int64_t c = kc + 8 * kq;
    const bool cin = c < k1;
    xf = buf_load16(xrs, cin ? (uint32_t)((tr * a.d + c) * 2) : kPastEnd, 0);
#pragma unroll
    for (int t = 0; t < ZTILES; ++t) {
      const int r = n0 + 16 * t + tr;
      af[t] = buf_load16(ars, (t < nt && cin && r < a.rank) ? (uint32_t)(((int64_t)r * a.d + c) * 2)
                                                             : kPastEnd, 0);
    }
  };
  u32x4 xa, xb, aa[ZTILES], ab[ZTILES];
  int64_t kc = k0;
  load(kc, xa, aa);
  while (kc < k1) {
    load(kc + 32, xb, ab);
#pragma unroll
    for (int t = 0; t < ZTILES; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, xa), __builtin_bit_cast(bf16x8, aa[t]), acc[t], 0, 0, 0);
    kc += 32;
    if (kc >= k1) break;
    load(kc + 32, xa, aa);
#pragma unroll
    for (int t = 0; t < ZTILES; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, xb), __builtin_bit_cast(bf16x8, ab[t]), acc[t], 0, 0, 0);
    kc += 32;
  }

  // waves in a fixed order; C of a 16x16 tile: lane l holds rank column
  // l & 15 and tokens 4 * (l >> 4) + i
  __shared__ float red[ZW][ZTILES * 4][64];
#pragma unroll
  for (int t = 0; t < ZTILES; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][t * 4 + i][l] = acc[t][i];
  __syncthreads();
  for (int e = tid; e < ZTILES * 4 * 64; e += ZW * 64) {
    const int ti = e >> 6, ll = e & 63;
    const int t = ti >> 2, i = ti & 3;
    const int64_t tok = m0 + 4 * (ll >> 4) + i;
    const int col = n0 + 16 * t + (ll & 15);
    if (t < nt && tok < a.M && col < a.rp) {
      const float v = ((red[0][ti][ll] + red[1][ti][ll]) + red[2][ti][ll]) + red[3][ti][ll];
      a.part[((int64_t)z * a.M + tok) * a.rp + col] = v;
    }
  }
}

__global__ __launch_bounds__(256) void k_lowrank_zsum(LowRankZArgs a, int nsplit) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = a.M * a.rp;
  if (i >= n) return;
  // slice order; the loads of 16 slices are in flight together
  float v = 0.f;
  for (int z0 = 0; z0 < nsplit; z0 += 16) {
    float t[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      t[j] = z0 + j < nsplit ? a.part[(int64_t)(z0 + j) * n + i] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (z0 + j < nsplit) v = (z0 + j == 0) ? t[j] : v + t[j];
  }
  a.Z[i] = (bf16_t)f2bf(v);
}

}  // namespace

// Channel slices of `slice` channels (256 for this kernel: a workgroup of 4
// waves x 64 channels; 128 for the partials the small-T statistics kernel
// writes, one 32-channel step per wave), fixed by d alone as long as the
// fp32 partials fit in 64 MiB: the slices and the order of their sum, hence
// every bit of a token's Z, then do not depend on how many tokens or
// requests share the launch.
int lowrank_z_splits(int64_t M, int64_t d, int rp, int slice) {
  int64_t s = (d + slice - 1) / slice;
  const int64_t per = (M > 0 ? M : 1) * (rp > 0 ? rp : 1) * (int64_t)sizeof(float);
  const int64_t cap = (int64_t(64) << 20) / per;
  if (s > cap) s = cap;
  return (int)(s < 1 ? 1 : s);
}

hipError_t launch_lowrank_z_small(const LowRankZArgs& a, const Launch& L) {
  if (a.M == 0) return hipSuccess;
  if (!a.part || a.rp % 32 != 0) return hipErrorInvalidValue;
  const int s = lowrank_z_splits(a.M, a.d, a.rp, 256);
  // slice length: a multiple of 128 channels (32 per wave)
  const int64_t kslice = ((a.d + s - 1) / s + 127) / 128 * 128;
  const dim3 grid((unsigned)((a.M + 15) / 16),
                  (unsigned)((a.rp + 16 * ZTILES - 1) / (16 * ZTILES)), (unsigned)s);
  return ext_launch(k_lowrank_zpart, grid, dim3(ZW * 64), 0, L, a, kslice);
}

hipError_t launch_lowrank_z_sum(const LowRankZArgs& a, int nsplit, const Launch& L) {
  const int64_t n = a.M * a.rp;
  if (n == 0) return hipSuccess;
  if (nsplit < 1) return hipErrorInvalidValue;
  return ext_launch(k_lowrank_zsum, dim3((unsigned)((n + 255) / 256)), dim3(256),
                    0, L, a, nsplit);
}

}  // namespace ttq
