// MFMA GEMM of the two-phase TTQ path on gfx950:
//
//   C[M][N] = A1[M][K1] * B1[N][K1]^T  +  A2[M][K2] * B2[N][K2]^T
//
// with bf16 operands, fp32 accumulation and fp32 (or bf16) output.  For the
// projection, A1 = X (tokens x channels), B1 = W_hat (weight rows x
// channels), and the optional second segment is the static low-rank term
// Z B^T with Z = X A^T ("TTQ: Activation-Aware Test-Time Quantization ...",
// gist.science zh summary, Sec. 2.2); the same kernel with one segment
// computes Z itself (split over K when the token count leaves too few output
// tiles to fill the chip; the fp32 partials are then summed in split order by
// a second small kernel).  Both operands are K-contiguous, which matches the
// v_mfma_f32_32x32x16_bf16 register layout (8 consecutive K values per lane).
//
// Tiling: 128 x 128 output tile per workgroup of 4 waves (2 x 2, each wave
// 64 x 64 = 2 x 2 MFMA tiles of 32 x 32), K step 64, both operand tiles
// double-buffered in LDS with a 16-byte row pad (conflict-free 16-byte
// reads).  With 8 or more weight tiles, workgroups are ordered so that the M
// tiles of one weight tile run back to back on the same XCD and share it
// through that XCD's L2; narrower outputs are spread over all XCDs.
#include "ttq_internal.h"

namespace ttq {

constexpr int GBM = 128, GBN = 128, GBK = 64, GLDK = GBK + 8;

__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs a) {
  if (a.nsplit > 1) {
    const int64_t kb = (int64_t)blockIdx.y * a.ksplit;
    a.A1 += kb;
    a.B1 += kb;
    a.K1 = min(a.ksplit, a.K1 - kb);
    a.C += (int64_t)blockIdx.y * a.split_stride;
  }
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][GBM * GLDK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][GBN * GLDK];

  const int64_t mtiles = (a.M + GBM - 1) / GBM;
  const int64_t ntiles = ((a.N > a.N_store ? a.N : a.N_store) + GBN - 1) / GBN;
  const int64_t id = blockIdx.x;
  int64_t ntile, mtile;
  if (ntiles >= 8) {
    const int xcd = (int)(id & 7);
    const int64_t j = id >> 3;
    ntile = (j / mtiles) * 8 + xcd;
    mtile = j % mtiles;
  } else {
    ntile = id % ntiles;
    mtile = id / ntiles;
  }
  if (ntile >= ntiles || mtile >= mtiles) return;
  const int64_t m0 = mtile * GBM, n0 = ntile * GBN;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const int64_t nk1 = (a.K1 + GBK - 1) / GBK;
  const int64_t nk2 = a.K2 > 0 ? (a.K2 + GBK - 1) / GBK : 0;
  const int64_t nk = nk1 + nk2;

  u32x4 ra[4], rb[4];
  auto load_regs = [&](int64_t kt) {
    const bool seg2 = kt >= nk1;
    const bf16_t* Ap = seg2 ? a.A2 : a.A1;
    const bf16_t* Bp = seg2 ? a.B2 : a.B1;
    const int64_t lda = seg2 ? a.lda2 : a.lda1;
    const int64_t ldb = seg2 ? a.ldb2 : a.ldb1;
    const int64_t K = seg2 ? a.K2 : a.K1;
    const int64_t k0 = (seg2 ? kt - nk1 : kt) * GBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cid = tid + 256 * i;
      const int r = cid >> 3;
      const int64_t k = k0 + (cid & 7) * 8;
      const int64_t m = m0 + r, n = n0 + r;
      ra[i] = (m < a.M && k < K) ? *(const u32x4*)(Ap + m * lda + k)
                                 : u32x4{0u, 0u, 0u, 0u};
      rb[i] = (n < a.N && k < K) ? *(const u32x4*)(Bp + n * ldb + k)
                                 : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cid = tid + 256 * i;
      const int r = cid >> 3, kc = (cid & 7) * 8;
      *(u32x4*)(&sA[buf][r * GLDK + kc]) = ra[i];
      *(u32x4*)(&sB[buf][r * GLDK + kc]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

  if (nk > 0) {
    load_regs(0);
    store_lds(0);
  }
  __syncthreads();
  const int fr = l & 31, fk = (l >> 5) * 8;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) load_regs(kt + 1);
#pragma unroll
    for (int kk = 0; kk < GBK / 16; ++kk) {
      u32x4 af[2], bfr[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[mt] = *(const u32x4*)(&sA[buf][(wm * 64 + mt * 32 + fr) * GLDK +
                                          kk * 16 + fk]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        bfr[nt] = *(const u32x4*)(&sB[buf][(wn * 64 + nt * 32 + fr) * GLDK +
                                           kk * 16 + fk]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, af[mt]),
              __builtin_bit_cast(bf16x8, bfr[nt]), acc[mt][nt], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // C layout of a 32x32 MFMA tile: lane l holds column l % 32 and rows
  // 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + mt * 32 + (r >> 2) * 8 + (l >> 5) * 4 +
                          (r & 3);
        const int64_t n = n0 + wn * 64 + nt * 32 + (l & 31);
        if (m < a.M && n < a.N_store) {
          if (a.C)
            a.C[m * a.ldc + n] = acc[mt][nt][r];
          else
            a.Cb[m * a.ldc + n] = (bf16_t)f2bf(acc[mt][nt][r]);
        }
      }
}

hipError_t launch_gemm(const GemmArgs& a, const Launch& L) {
  const int64_t mtiles = (a.M + GBM - 1) / GBM;
  const int64_t ntiles = ((a.N > a.N_store ? a.N : a.N_store) + GBN - 1) / GBN;
  const int64_t nblk =
      ntiles >= 8 ? ((ntiles + 7) / 8) * 8 * mtiles : ntiles * mtiles;
  if (nblk == 0) return hipSuccess;
  const unsigned ns = a.nsplit > 1 ? (unsigned)a.nsplit : 1u;
  return ext_launch(k_gemm, dim3((unsigned)nblk, ns), dim3(256), 0, L, a);
}

__global__ __launch_bounds__(256) void k_splitk_reduce(SplitReduceArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= a.n) return;
  f32x4 acc = *(const f32x4*)(a.part + i);
  for (int z = 1; z < a.nsplit; ++z) {
    const f32x4 v = *(const f32x4*)(a.part + (int64_t)z * a.n + i);
    acc[0] += v[0];
    acc[1] += v[1];
    acc[2] += v[2];
    acc[3] += v[3];
  }
  u32x2 o;
  o.x = pack_bf16(acc[0], acc[1]);
  o.y = pack_bf16(acc[2], acc[3]);
  *(u32x2*)(a.out + i) = o;
}

hipError_t launch_splitk_reduce(const SplitReduceArgs& a, const Launch& L) {
  if (a.n == 0) return hipSuccess;
  const int64_t nthr = (a.n + 3) / 4;
  return ext_launch(k_splitk_reduce, dim3((unsigned)((nthr + 255) / 256)),
                    dim3(256), 0, L, a);
}

}  // namespace ttq
