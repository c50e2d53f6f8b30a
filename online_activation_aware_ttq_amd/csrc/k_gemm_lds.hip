// Large-tile MFMA GEMM of the two-phase TTQ path on gfx950:
//
//   C[M][N] = A1[M][K1] * B1[N][K1]^T  +  A2[M][K2] * B2[N][K2]^T   (fp32 C)
//
// For the projection A1 = X (tokens x channels), B1 = W_hat (dequantized
// weight rows, D^{-1/2} folded in) and the second segment is the static
// low-rank term Z B^T with Z = X A^T ("TTQ: Activation-Aware Test-Time
// Quantization ...", gist.science zh summary, Sec. 2.2).  Both operands are
// K-contiguous, the layout v_mfma_f32_32x32x16_bf16 reads (8 consecutive K
// values per lane).
//
// Data movement (CDNA4):
//  * operand tiles go from global memory straight into LDS with
//    buffer_load_dwordx4 ... lds (no staging registers, no ds_write).  One
//    wave instruction fills 1 KB = 8 rows x 128 bytes (64 channels).  A
//    buffer descriptor bounds each operand tile, so rows past M / N and
//    channels past K read as zeros with no memory traffic;
//  * inside a 128-byte LDS row the eight 16-byte chunks are XOR-swizzled so
//    that the 32-row fragment reads of an MFMA operand are conflict-free;
//  * NS stages of 64 channels; the loads for tile kt+NS are issued right
//    after the barrier that retires tile kt, interleaved one or two at a
//    time between the MFMAs of that step (a burst of LDS-DMA instructions
//    stalls the issuing wave; spread out they hide behind the matrix core);
//  * fragment reads for the next 16-channel step are interleaved with the
//    MFMAs of the current one (register double buffer).
// Workgroups are ordered so that the M tiles of one weight tile run back to
// back on the same XCD (shared through that XCD's L2); narrower outputs are
// spread over all XCDs.  A batch of independent products (one per request,
// each with its own W_hat) is the second grid dimension.
#include "ttq_internal.h"

namespace ttq {

namespace {

// physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r):
// conflict-free 16-byte reads of 8 and of 16 consecutive rows
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// TM x TN MFMA tiles of 32 x 32 per wave, WGM x WGN waves, NS LDS stages.
template <int TM, int TN, int WGM, int WGN, int NS>
__global__ __launch_bounds__(WGM * WGN * 64, 1) void k_gemm_lds(GemmArgs a) {
  if (blockIdx.y > 0) {  // product z of a batch
    const int64_t z = blockIdx.y;
    a.A1 += z * a.sA1;
    a.B1 += z * a.sB1;
    if (a.A2) a.A2 += z * a.sA2;
    if (a.B2) a.B2 += z * a.sB2;
    a.C += z * a.sC;
  }
  constexpr int NW = WGM * WGN;
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32, BK = 64;
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2;
  constexpr int STAGE = ABYTES + BBYTES;
  constexpr int NLA = BM / (8 * NW), NLB = BN / (8 * NW);  // loads / tile / wave
  constexpr int NL = NLA + NLB;
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "load split");
  static_assert(NW % 2 == 0, "row parity of a wave's load rows");
  static_assert(NS >= 2 && (NS - 2) * NL < 64, "stages");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int64_t mtiles = (a.M + BM - 1) / BM;
  const int64_t ntiles = (a.N_store + BN - 1) / BN;
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
  const int64_t m0 = mtile * BM, n0 = ntile * BN;
  const int64_t mrows = min((int64_t)BM, a.M - m0);
  const int64_t nrows = max((int64_t)0, min((int64_t)BN, a.N - n0));

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WGN, wn = w % WGN;

  // loads: wave w, instruction j fills rows (w + j*NW)*8 .. +8; lane l
  // writes row +l/8, physical chunk l%8, i.e. logical chunk (l%8)^swz(row);
  // the row parity is that of w (NW even), so the chunk is fixed per lane
  const int lrow = l >> 3;
  const int lch = (l & 7) ^ swz(w * 8 + lrow);
  const int nk1 = (int)((a.K1 + BK - 1) / BK);
  const int nk2 = a.K2 > 0 ? (int)((a.K2 + BK - 1) / BK) : 0;
  const int nk = nk1 + nk2;

  // Tiles at or past nk read nothing: both segments put every lane out of
  // range (zero fill into a stage that is not read again).
  auto issue = [&](int kt, int stage) {
    const bool seg2 = kt >= nk1;
    const bf16_t* Ap = seg2 ? a.A2 : a.A1;
    const bf16_t* Bp = seg2 ? a.B2 : a.B1;
    const int lda = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.lda2 : a.lda1));
    const int ldb = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.ldb2 : a.ldb1));
    const int K = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.K2 : a.K1));
    const int k0 = __builtin_amdgcn_readfirstlane((seg2 ? kt - nk1 : kt) * BK);
    const auto ra = make_rsrc(Ap + m0 * lda, (uint32_t)(mrows * lda * 2));
    const auto rb = make_rsrc(Bp + n0 * ldb, (uint32_t)(nrows * ldb * 2));
    const bool kin = k0 + lch * 8 < K;
    const uint32_t va =
        kin ? (uint32_t)(((w * 8 + lrow) * lda + k0 + lch * 8) * 2) : kOutOfRange;
    const uint32_t vb =
        kin ? (uint32_t)(((w * 8 + lrow) * ldb + k0 + lch * 8) * 2) : kOutOfRange;
    unsigned char* sa = smem + stage * STAGE;
    unsigned char* sb = sa + ABYTES;
#pragma unroll
    for (int j = 0; j < NLA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(sa + (w + j * NW) * 1024),
          16, va, (uint32_t)(j * 8 * NW * lda * 2), 0, 0);
#pragma unroll
    for (int j = 0; j < NLB; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(sb + (w + j * NW) * 1024),
          16, vb, (uint32_t)(j * 8 * NW * ldb * 2), 0, 0);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment reads: lane l reads row l%32 of each 32-row tile, logical chunk
  // 2*kk + l/32; swz(row) depends on l%16 only
  const int fs = swz(l & 15);
  const int fh = l >> 5;
  const int arow = (wm * TM * 32 + (l & 31)) * 128;
  const int brow = (wn * TN * 32 + (l & 31)) * 128;
  u32x4 fa[2][TM], fb[2][TN];
  auto read_frags = [&](int stage, int kk, u32x4* A_, u32x4* B_) {
    const unsigned char* sa = smem + stage * STAGE;
    const unsigned char* sb = sa + ABYTES;
    const int off = (((kk << 1) | fh) ^ fs) * 16;
#pragma unroll
    for (int j = 0; j < TN; ++j) B_[j] = *(const u32x4*)(sb + brow + j * 4096 + off);
#pragma unroll
    for (int i = 0; i < TM; ++i) A_[i] = *(const u32x4*)(sa + arow + i * 4096 + off);
  };
  auto mfmas = [&](const u32x4* A_, const u32x4* B_) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, A_[i]), __builtin_bit_cast(bf16x8, B_[j]),
            acc[i][j], 0, 0, 0);
  };

  // prologue: tiles 0 .. NS-2 in flight, wait for tile 0
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p, p);
  wait_vm<(NS - 2) * NL>();
  lds_barrier();
  read_frags(0, 0, fa[0], fb[0]);
  issue(NS - 1, NS - 1);

  constexpr int NMF = TM * TN;
  constexpr int PR = (TM + TN + NMF - 1) / NMF;   // fragment reads per MFMA
  constexpr int PL = (NL + NMF - 1) / NMF;        // tile loads per MFMA
  int stage = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int nstage = stage + 1 == NS ? 0 : stage + 1;
#pragma unroll
    for (int kk = 0; kk < BK / 16 - 1; ++kk) {
      const int cur = kk & 1;
      read_frags(stage, kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
      mfmas(fa[cur], fb[cur]);
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, PR, 0);  // DS read
      }
    }
    {
      constexpr int cur = (BK / 16 - 1) & 1;
      // tile kt+1 landed (NS-2 younger tiles may still be in flight)
      wait_vm<(NS - 2) * NL>();
      lds_barrier();   // ... for every wave; all reads of stage kt done
      read_frags(nstage, 0, fa[cur ^ 1], fb[cur ^ 1]);
      issue(kt + NS, stage);
      mfmas(fa[cur], fb[cur]);
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, PR, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x020, PL, 0);  // VMEM read
      }
    }
    stage = nstage;
  }
  // the loads issued past the last tile read nothing, but they still write
  // LDS: let them retire before the workgroup ends
  wait_vm<0>();

  // C layout of a 32x32 MFMA tile: lane l holds column l%32 and rows
  // 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m =
            m0 + wm * TM * 32 + i * 32 + (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
        const int64_t n = n0 + wn * TN * 32 + j * 32 + (l & 31);
        if (m < a.M && n < a.N_store) a.C[m * a.ldc + n] = acc[i][j][r];
      }
}

template <int TM, int TN, int WGM, int WGN, int NS>
hipError_t launch_t(const GemmArgs& a, const Launch& L) {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  constexpr int lds = NS * (BM + BN) * 64 * 2;
  static_assert(lds <= 160 * 1024, "LDS");
  const int64_t mtiles = (a.M + BM - 1) / BM;
  const int64_t ntiles = (a.N_store + BN - 1) / BN;
  const int64_t nblk =
      ntiles >= 8 ? ((ntiles + 7) / 8) * 8 * mtiles : ntiles * mtiles;
  if (nblk == 0) return hipSuccess;
  // more than 64 KB of dynamic LDS must be allowed per kernel (idempotent)
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(k_gemm_lds<TM, TN, WGM, WGN, NS>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const unsigned nb = a.batch > 1 ? (unsigned)a.batch : 1u;
  return ext_launch(k_gemm_lds<TM, TN, WGM, WGN, NS>, dim3((unsigned)nblk, nb),
                    dim3(WGM * WGN * 64), lds, L, a);
}

}  // namespace

int gemm_lds_config(int64_t M, int64_t N, int64_t batch) {
  // 256 x 256 tiles keep the most MFMA work per LDS byte; when they would
  // leave a quarter of the 256 CUs idle in a single round, 256 x 128 tiles
  // give twice as many workgroups
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256) * batch;
  return big >= 192 ? 0 : 1;
}

hipError_t launch_gemm_lds(const GemmArgs& a, const Launch& L) {
  if (a.M <= 0 || a.N_store <= 0) return hipSuccess;
  if (a.K1 <= 0 || !a.C || a.nsplit > 1) return hipErrorInvalidValue;
  if (gemm_lds_config(a.M, a.N_store, a.batch > 1 ? a.batch : 1) == 0)
    return launch_t<4, 2, 2, 4, 2>(a, L);   // 256 x 256, 8 waves, 2 stages
  return launch_t<2, 2, 4, 2, 3>(a, L);     // 256 x 128, 8 waves, 3 stages
}

}  // namespace ttq
