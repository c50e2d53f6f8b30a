// First factor of the static low-rank term of TTQ for small token counts:
//   Z[m][k] = sum_j X[m][j] * A[k][j]       (Z = X A^T, i.e. (A X)^T)
// ("TTQ: Activation-Aware Test-Time Quantization ...", gist.science zh
// summary, Sec. 2.2: W ~ W_q + B A with static B, A).  Stored as bf16 with the
// rank padded to a multiple of 32 (zeros), the operand layout the fused
// kernel's MFMA tail reads.  A workgroup computes one rank index for up to 16
// tokens: lanes stride over the channels with 16-byte loads, the partial
// dot products are reduced across the workgroup in a fixed order.
#include "ttq_internal.h"

namespace ttq {

__global__ __launch_bounds__(256) void k_lowrank_z(LowRankZArgs a) {
  constexpr int TM = 16;
  const int k = blockIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int mcount = (int)min((int64_t)TM, a.M - m0);
  if (k >= a.rank) {
    if (tid < mcount) a.Z[(m0 + tid) * a.rp + k] = 0;
    return;
  }
  float acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] = 0.f;
  const bf16_t* Ak = a.A + (int64_t)k * a.d;
  for (int64_t c = (int64_t)tid * 8; c < a.d; c += 2048) {
    const u32x4 av = *(const u32x4*)(Ak + c);
    const float af[8] = {bf16lo(av.x), bf16hi(av.x), bf16lo(av.y),
                         bf16hi(av.y), bf16lo(av.z), bf16hi(av.z),
                         bf16lo(av.w), bf16hi(av.w)};
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i < mcount) {
        const u32x4 xv = *(const u32x4*)(a.X + (m0 + i) * a.d + c);
        float s = acc[i];
        s = fmaf(bf16lo(xv.x), af[0], s);
        s = fmaf(bf16hi(xv.x), af[1], s);
        s = fmaf(bf16lo(xv.y), af[2], s);
        s = fmaf(bf16hi(xv.y), af[3], s);
        s = fmaf(bf16lo(xv.z), af[4], s);
        s = fmaf(bf16hi(xv.z), af[5], s);
        s = fmaf(bf16lo(xv.w), af[6], s);
        s = fmaf(bf16hi(xv.w), af[7], s);
        acc[i] = s;
      }
    }
  }
  __shared__ float red[4][TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float v = acc[i];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (l == 0) red[w][i] = v;
  }
  __syncthreads();
  if (tid < mcount) {
    const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    a.Z[(m0 + tid) * a.rp + k] = (bf16_t)f2bf(v);
  }
}

hipError_t launch_lowrank_z_small(const LowRankZArgs& a, const Launch& L) {
  if (a.M == 0) return hipSuccess;
  dim3 grid((unsigned)a.rp, (unsigned)((a.M + 15) / 16));
  return ext_launch(k_lowrank_z, grid, dim3(256), 0, L, a);
}

}  // namespace ttq
