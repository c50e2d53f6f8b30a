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
// Tile order: the output tiles of all products of the batch are laid out in
// strips of 8 N tiles (row by row inside a strip).  With one tile per
// workgroup (fewer than four rounds of tiles) each of the 8 XCDs (workgroups
// id, id + 8, ...) takes one contiguous eighth of that order, so that the ~32
// workgroups an XCD runs at once cover a patch of about 4 M x 8 N tiles whose
// operand slices its L2 shares, and a partial last round is spread evenly
// over the XCDs; the persistent kernel deals 32-tile patches round-robin to
// the XCDs instead (see there).  Operand loads carry the device-scope cache
// bit (sc0; measured slightly faster than the default here).
#include "ttq_internal.h"

#include <algorithm>
#include <numeric>

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

// strip width of the tile order (N tiles)
constexpr int kStripN = 8;

// Step schedules (SCHED):
//  kDoubleBuf: fragments for the next 16-channel step are read while the
//    current one is contracted (two register sets); the loads of tile kt+NS
//    go out after the barrier in the last step of tile kt;
//  kSingleBuf: one register set, each step reads its fragments and then
//    contracts them; the loads of tile kt+NS-1 are spread over the MFMAs of
//    the first step of tile kt, right after the barrier that retired the
//    stage they overwrite;
//  kSingleBufSplit: the same, with the A loads in the first step and the B
//    loads in the second.
// Every schedule runs the same MFMAs in the same order on every output, so
// the result does not depend on it.  Measured (256 x 256 tiles): with many
// rounds of workgroups per CU (7B-class layer, 8 requests x 4096 tokens)
// kSingleBuf takes 6-9 % less time than kDoubleBuf, and in the persistent
// kernel below kSingleBufSplit another 2-4 % less; with one partial round
// (70B-class up projection, T = 512) kSingleBuf is 15 % slower and
// kSingleBufSplit 4 % faster than kDoubleBuf.
constexpr int kDoubleBuf = 0, kSingleBuf = 1, kSingleBufSplit = 2;

// TM x TN MFMA tiles of 32 x 32 per wave, WGM x WGN waves, NS LDS stages.
template <int TM, int TN, int WGM, int WGN, int NS, int SCHED>
__global__ __launch_bounds__(WGM * WGN * 64, 1) void k_gemm_lds(GemmArgs a) {
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
  const int64_t per_product = mtiles * ntiles;
  const int64_t nprod = a.batch > 1 ? a.batch : 1;
  const int64_t total = per_product * nprod;
  // this XCD's contiguous share of the tile order, then the tile
  const int64_t xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int64_t base = total >> 3, extra = total & 7;
  if (j >= base + (xcd < extra ? 1 : 0)) return;
  const int64_t t = xcd * base + min(xcd, extra) + j;
  const int64_t z = t / per_product, tz = t % per_product;
  const int64_t strip = tz / (kStripN * mtiles), in_strip = tz % (kStripN * mtiles);
  const int64_t width = min((int64_t)kStripN, ntiles - strip * kStripN);
  const int64_t mtile = in_strip / width;
  const int64_t ntile = strip * kStripN + in_strip % width;
  if (z > 0) {  // product z of a batch
    a.A1 += z * a.sA1;
    a.B1 += z * a.sB1;
    if (a.A2) a.A2 += z * a.sA2;
    if (a.B2) a.B2 += z * a.sB2;
    a.C += z * a.sC;
  }
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
  // part: 1 = A loads, 2 = B loads, 3 = both
  auto issue = [&](int kt, int stage, int part) {
    const bool seg2 = kt >= nk1;
    const bf16_t* Ap = seg2 ? a.A2 : a.A1;
    const bf16_t* Bp = seg2 ? a.B2 : a.B1;
    const int lda = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.lda2 : a.lda1));
    const int ldb = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.ldb2 : a.ldb1));
    const int K = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.K2 : a.K1));
    const int k0 = __builtin_amdgcn_readfirstlane((seg2 ? kt - nk1 : kt) * BK);
    const auto ra = make_rsrc(Ap + m0 * lda, (uint32_t)(mrows * lda * 2));
    const bool kin = k0 + lch * 8 < K;
    const uint32_t va =
        kin ? (uint32_t)(((w * 8 + lrow) * lda + k0 + lch * 8) * 2) : kOutOfRange;
    // B1 in the tiled W_hat layout: this tile's rows are rows n0 % 256 ..
    // of 256-row block n0 / 256, whose k-tiles are contiguous 32 KiB tiles
    const bool tiled = a.b1_tiled && !seg2;
    const auto rb =
        tiled ? make_rsrc(Bp + (n0 / kWtRows) * nk1 * (kWtRows * kWtCols),
                          (uint32_t)(nk1 * (kWtRows * kWtCols) * 2))
              : make_rsrc(Bp + n0 * ldb, (uint32_t)(nrows * ldb * 2));
    const uint32_t vb =
        !kin ? kOutOfRange
             : tiled ? (uint32_t)(((kt * kWtRows + n0 % kWtRows + w * 8 + lrow) * kWtCols +
                                   lch * 8) * 2)
                     : (uint32_t)(((w * 8 + lrow) * ldb + k0 + lch * 8) * 2);
    const int ldbs = tiled ? (int)kWtCols : ldb;   // row step of the B loads
    unsigned char* sa = smem + stage * STAGE;
    unsigned char* sb = sa + ABYTES;
    if (part & 1) {
#pragma unroll
      for (int j = 0; j < NLA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(sa + (w + j * NW) * 1024),
            16, va, (uint32_t)(j * 8 * NW * lda * 2), 0, 1);
    }
    if (part & 2) {
#pragma unroll
      for (int j = 0; j < NLB; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(sb + (w + j * NW) * 1024),
            16, vb, (uint32_t)(j * 8 * NW * ldbs * 2), 0, 1);
    }
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

  constexpr int NMF = TM * TN;
  if constexpr (SCHED == kDoubleBuf) {
    u32x4 fa[2][TM], fb[2][TN];
    // prologue: tiles 0 .. NS-2 in flight, wait for tile 0
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) issue(p, p, 3);
    wait_vm<(NS - 2) * NL>();
    lds_barrier();
    read_frags(0, 0, fa[0], fb[0]);
    issue(NS - 1, NS - 1, 3);

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
        issue(kt + NS, stage, 3);
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
  } else {
    u32x4 fa[TM], fb[TN];
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) issue(p, p, 3);
    wait_vm<(NS - 2) * NL>();
    lds_barrier();
    constexpr int PL = (NL + NMF - 1) / NMF;
    constexpr int PA = (NLA + NMF - 1) / NMF, PB = (NLB + NMF - 1) / NMF;
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
      // the stage tile kt-1 used was retired by the last barrier
      const int pstage = stage == 0 ? NS - 1 : stage - 1;
      if constexpr (SCHED == kSingleBuf) {
        read_frags(stage, 0, fa, fb);
        issue(kt + NS - 1, pstage, 3);
        mfmas(fa, fb);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, PL, 0);  // VMEM read
        }
      } else {
        read_frags(stage, 0, fa, fb);
        issue(kt + NS - 1, pstage, 1);
        mfmas(fa, fb);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, PA, 0);
        }
        read_frags(stage, 1, fa, fb);
        issue(kt + NS - 1, pstage, 2);
        mfmas(fa, fb);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, PB, 0);
        }
      }
#pragma unroll
      for (int kk = SCHED == kSingleBuf ? 1 : 2; kk < BK / 16; ++kk) {
        read_frags(stage, kk, fa, fb);
        mfmas(fa, fb);
      }
      // tile kt+1 landed (NS-2 younger tiles may still be in flight), and
      // every wave is done with this stage
      wait_vm<(NS - 2) * NL>();
      lds_barrier();
      stage = stage + 1 == NS ? 0 : stage + 1;
    }
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

// Persistent form of the single-buffered schedules: one workgroup per CU
// walks its XCD's share of the tile order.  Measured on the 7B-class
// layer (8 requests x 4096 tokens), split-load schedule, alternating runs:
// q 1205 -> 1034 us, gate 2981 -> 2742, down 2781 -> 2550; one partial
// round (T = 512) gains nothing, so fewer than four rounds keep one tile
// per workgroup.  At the end of a tile the
// loads of the next tile's first k-tiles go out first, then C leaves through
// LDS (32-row passes through the free stage, one 16-byte store per lane and
// row piece, 1 KiB per wave instruction) and the next tile's k-loop starts
// while those stores drain.  With one workgroup per CU (LDS) the C stores
// of a tile otherwise stall the CU: every round of tiles ends in the same
// store burst, bound by the write bandwidth (timing copy without the C
// stores: 10-20 % faster on the 7B-class layer).  The MFMAs and their order
// per output are those of k_gemm_lds: the results are bit-identical.
template <int TM, int TN, int WGM, int WGN, int NS, int SCHED>
__global__ __launch_bounds__(WGM * WGN * 64, 1) void k_gemm_lds_p(GemmArgs a) {
  constexpr int NW = WGM * WGN, NT = NW * 64;
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32, BK = 64;
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2;
  constexpr int STAGE = ABYTES + BBYTES;
  constexpr int NLA = BM / (8 * NW), NLB = BN / (8 * NW);
  constexpr int NL = NLA + NLB;
  constexpr int CST = BN + 4;                    // staged C row (floats)
  constexpr int NSTORE = BM * BN / 4 / NT;       // 16-byte stores per thread
  static_assert(SCHED != kDoubleBuf, "single-buffered schedules only");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0 && NW % 2 == 0, "load split");
  static_assert(NS == 2, "one k-tile of the next tile in flight during the C stores");
  static_assert(NSTORE + (NS - 2) * NL < 64, "vmcnt range");
  static_assert(32 * CST * 4 <= STAGE, "C pass fits a stage");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int64_t mtiles = (a.M + BM - 1) / BM;
  const int64_t ntiles = (a.N_store + BN - 1) / BN;
  const int64_t per_product = mtiles * ntiles;
  const int64_t nprod = a.batch > 1 ? a.batch : 1;
  const int64_t total = per_product * nprod;
  // the tile order is cut in chunks of 32 consecutive tiles (a 4 x 8 patch of
  // one product), dealt round-robin to the XCDs: XCD x takes chunks x, x + 8,
  // ..., and its workgroup jj the tiles jj, jj + nper, ... of that list
  // (blocks of one XCD are id, id + 8, ...).  With 32 CUs per XCD all XCDs
  // then work on the same product at a time, so the last-level cache holds
  // one product's operands instead of eight (measured on the 7B-class layer
  // against contiguous eighths per XCD: q 1130 -> 1015 us, gate 2770 ->
  // 2420, down 2620 -> 2355).
  const int64_t xcd = blockIdx.x & 7, jj = blockIdx.x >> 3, nper = gridDim.x >> 3;
  const int64_t full = total / 256, rem = total % 256;
  const int64_t cnt = full * 32 + min((int64_t)32, max((int64_t)0, rem - xcd * 32));
  if (jj >= cnt) return;

  // the current tile (plain locals: a local struct used inside the load
  // lambda keeps the compiler from emitting this kernel's host stub)
  const bf16_t *tA1 = nullptr, *tB1 = nullptr, *tA2 = nullptr, *tB2 = nullptr;
  float* tC = nullptr;
  int64_t tm0 = 0, tn0 = 0, tmrows = 0, tnrows = 0;
  auto set_tile = [&](int64_t j) {
    const int64_t t = (xcd + 8 * (j / 32)) * 32 + (j % 32);
    const int64_t z = t / per_product, tz = t % per_product;
    const int64_t strip = tz / (kStripN * mtiles), in_strip = tz % (kStripN * mtiles);
    const int64_t width = min((int64_t)kStripN, ntiles - strip * kStripN);
    tm0 = (in_strip / width) * BM;
    tn0 = (strip * kStripN + in_strip % width) * BN;
    tA1 = a.A1 + z * a.sA1;
    tB1 = a.B1 + z * a.sB1;
    tA2 = a.A2 ? a.A2 + z * a.sA2 : nullptr;
    tB2 = a.B2 ? a.B2 + z * a.sB2 : nullptr;
    tC = a.C + z * a.sC;
    tmrows = min((int64_t)BM, a.M - tm0);
    tnrows = max((int64_t)0, min((int64_t)BN, a.N - tn0));
  };

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WGN, wn = w % WGN;
  const int lrow = l >> 3;
  const int lch = (l & 7) ^ swz(w * 8 + lrow);
  const int nk1 = (int)((a.K1 + BK - 1) / BK);
  const int nk2 = a.K2 > 0 ? (int)((a.K2 + BK - 1) / BK) : 0;
  const int nk = nk1 + nk2;

  // loads of k-tile kt of the current tile (tiles at or past nk read
  // nothing: zero fill into a stage not read again)
  set_tile(jj);
  auto issue = [&](int kt, int stage, int part) {
    const bool seg2 = kt >= nk1;
    const bf16_t* Ap = seg2 ? tA2 : tA1;
    const bf16_t* Bp = seg2 ? tB2 : tB1;
    const int lda = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.lda2 : a.lda1));
    const int ldb = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.ldb2 : a.ldb1));
    const int K = __builtin_amdgcn_readfirstlane((int)(seg2 ? a.K2 : a.K1));
    const int k0 = __builtin_amdgcn_readfirstlane((seg2 ? kt - nk1 : kt) * BK);
    const auto ra = make_rsrc(Ap + tm0 * lda, (uint32_t)(tmrows * lda * 2));
    const bool kin = k0 + lch * 8 < K;
    const uint32_t va =
        kin ? (uint32_t)(((w * 8 + lrow) * lda + k0 + lch * 8) * 2) : kOutOfRange;
    // B1 in the tiled W_hat layout (see k_gemm_lds)
    const bool tiled = a.b1_tiled && !seg2;
    const auto rb =
        tiled ? make_rsrc(Bp + (tn0 / kWtRows) * nk1 * (kWtRows * kWtCols),
                          (uint32_t)(nk1 * (kWtRows * kWtCols) * 2))
              : make_rsrc(Bp + tn0 * ldb, (uint32_t)(tnrows * ldb * 2));
    const uint32_t vb =
        !kin ? kOutOfRange
             : tiled ? (uint32_t)(((kt * kWtRows + tn0 % kWtRows + w * 8 + lrow) * kWtCols +
                                   lch * 8) * 2)
                     : (uint32_t)(((w * 8 + lrow) * ldb + k0 + lch * 8) * 2);
    const int ldbs = tiled ? (int)kWtCols : ldb;   // row step of the B loads
    unsigned char* sa = smem + stage * STAGE;
    unsigned char* sb = sa + ABYTES;
    if (part & 1) {
#pragma unroll
      for (int j = 0; j < NLA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(sa + (w + j * NW) * 1024),
            16, va, (uint32_t)(j * 8 * NW * lda * 2), 0, 1);
    }
    if (part & 2) {
#pragma unroll
      for (int j = 0; j < NLB; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(sb + (w + j * NW) * 1024),
            16, vb, (uint32_t)(j * 8 * NW * ldbs * 2), 0, 1);
    }
  };

  const int fs = swz(l & 15);
  const int fh = l >> 5;
  const int arow = (wm * TM * 32 + (l & 31)) * 128;
  const int brow = (wn * TN * 32 + (l & 31)) * 128;
  auto read_frags = [&](int stage, int kk, u32x4* A_, u32x4* B_) {
    const unsigned char* sa = smem + stage * STAGE;
    const unsigned char* sb = sa + ABYTES;
    const int off = (((kk << 1) | fh) ^ fs) * 16;
#pragma unroll
    for (int j = 0; j < TN; ++j) B_[j] = *(const u32x4*)(sb + brow + j * 4096 + off);
#pragma unroll
    for (int i = 0; i < TM; ++i) A_[i] = *(const u32x4*)(sa + arow + i * 4096 + off);
  };
  f32x16 acc[TM][TN];
  auto mfmas = [&](const u32x4* A_, const u32x4* B_) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, A_[i]), __builtin_bit_cast(bf16x8, B_[j]),
            acc[i][j], 0, 0, 0);
  };
  constexpr int NMF = TM * TN;
  constexpr int PL = (NL + NMF - 1) / NMF;
  constexpr int PA = (NLA + NMF - 1) / NMF, PB = (NLB + NMF - 1) / NMF;
  const bool cvec = (a.ldc % 4 == 0) && (a.sC % 4 == 0) &&
                    ((reinterpret_cast<uintptr_t>(a.C) & 15) == 0);

  issue(0, 0, 3);
  wait_vm<0>();
  for (int64_t j = jj; j < cnt; j += nper) {
    // k-tile 0 of this tile landed (the previous tile's C stores, issued
    // after it, may still be in flight)
    wait_vm<NSTORE>();
    lds_barrier();
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jn = 0; jn < TN; ++jn)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.f;
    u32x4 fa[TM], fb[TN];
    int stage = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const int pstage = stage == 0 ? NS - 1 : stage - 1;
      if constexpr (SCHED == kSingleBuf) {
        read_frags(stage, 0, fa, fb);
        issue(kt + NS - 1, pstage, 3);
        mfmas(fa, fb);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, PL, 0);  // VMEM read
        }
      } else {
        read_frags(stage, 0, fa, fb);
        issue(kt + NS - 1, pstage, 1);
        mfmas(fa, fb);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, PA, 0);
        }
        read_frags(stage, 1, fa, fb);
        issue(kt + NS - 1, pstage, 2);
        mfmas(fa, fb);
#pragma unroll
        for (int q = 0; q < NMF; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, PB, 0);
        }
      }
#pragma unroll
      for (int kk = SCHED == kSingleBuf ? 1 : 2; kk < BK / 16; ++kk) {
        read_frags(stage, kk, fa, fb);
        mfmas(fa, fb);
      }
      wait_vm<(NS - 2) * NL>();
      lds_barrier();
      stage = stage + 1 == NS ? 0 : stage + 1;
    }
    // the loads issued past the last k-tile still write LDS
    wait_vm<0>();
    lds_barrier();
    // the next tile's first k-tile goes out before the C stores
    const int64_t om0 = tm0, on0 = tn0;
    float* oC = tC;
    if (j + nper < cnt) {
      set_tile(j + nper);
      issue(0, 0, 3);
    }
    // C through the second stage, 32 rows per pass: the waves holding those
    // rows write their 32 x 32 fragments (lane l: column l%32, rows
    // 8*(r/4) + 4*(l/32) + r%4), then every thread stores 16-byte pieces of
    // whole rows
    float* cs = reinterpret_cast<float*>(smem + (NS - 1) * STAGE);
#pragma unroll
    for (int p = 0; p < BM / 32; ++p) {
      if (wm == p / TM) {
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
            cs[row * CST + wn * TN * 32 + jn * 32 + (l & 31)] = acc[p % TM][jn][r];
          }
      }
      lds_barrier();
#pragma unroll
      for (int e = 0; e < 32 * BN / 4 / NT; ++e) {
        const int idx = tid + e * NT;
        const int row = idx / (BN / 4), c4 = idx % (BN / 4);
        const f32x4 v = *(const f32x4*)(cs + row * CST + c4 * 4);
        const int64_t m = om0 + p * 32 + row, n = on0 + c4 * 4;
        if (m < a.M) {
          float* dst = oC + m * a.ldc + n;
          if (cvec && n + 3 < a.N_store) {
            *(f32x4*)dst = v;
          } else {
            if (n < a.N_store) dst[0] = v.x;
            if (n + 1 < a.N_store) dst[1] = v.y;
            if (n + 2 < a.N_store) dst[2] = v.z;
            if (n + 3 < a.N_store) dst[3] = v.w;
          }
        }
      }
      lds_barrier();
    }
  }
}

template <int TM, int TN, int WGM, int WGN, int NS, int SCHED>
hipError_t launch_t(const GemmArgs& a, const Launch& L) {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  constexpr int lds = NS * (BM + BN) * 64 * 2;
  static_assert(lds <= 160 * 1024, "LDS");
  const int64_t mtiles = (a.M + BM - 1) / BM;
  const int64_t ntiles = (a.N_store + BN - 1) / BN;
  const int64_t total = mtiles * ntiles * (a.batch > 1 ? a.batch : 1);
  const int64_t nblk = (total + 7) / 8 * 8;
  if (nblk == 0) return hipSuccess;
  // more than 64 KB of dynamic LDS must be allowed per kernel (idempotent)
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(k_gemm_lds<TM, TN, WGM, WGN, NS, SCHED>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  return ext_launch(k_gemm_lds<TM, TN, WGM, WGN, NS, SCHED>, dim3((unsigned)nblk),
                    dim3(WGM * WGN * 64), lds, L, a);
}

// persistent launch: one workgroup per CU (at most), a multiple of 8
template <int TM, int TN, int WGM, int WGN, int NS, int SCHED>
hipError_t launch_tp(const GemmArgs& a, const Launch& L) {
  constexpr int BM = WGM * TM * 32, BN = WGN * TN * 32;
  constexpr int lds = NS * (BM + BN) * 64 * 2;
  static_assert(lds <= 160 * 1024, "LDS");
  const int64_t mtiles = (a.M + BM - 1) / BM;
  const int64_t ntiles = (a.N_store + BN - 1) / BN;
  const int64_t total = mtiles * ntiles * (a.batch > 1 ? a.batch : 1);
  if (total == 0) return hipSuccess;
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = n > 0 ? n : 256;
  }
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t wg_xcd = std::min<int64_t>(per_xcd, std::max(1, cus / 8));
  static hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(k_gemm_lds_p<TM, TN, WGM, WGN, NS, SCHED>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  return ext_launch(k_gemm_lds_p<TM, TN, WGM, WGN, NS, SCHED>,
                    dim3((unsigned)(wg_xcd * 8)), dim3(WGM * WGN * 64), lds, L, a);
}

}  // namespace

int gemm_lds_config(int64_t M, int64_t N, int64_t batch) {
  // 256 x 256 tiles move the fewest operand bytes per flop; 256 x 128 tiles
  // give twice as many workgroups, each costing about 0.57 of a big one
  // (measured on the 7B-class shapes).  Take the one whose rounds of 256
  // workgroups (one per CU) cost less: a partial last round costs a full one.
  // From four rounds of 256 x 256 tiles on, one persistent workgroup per CU
  // walks the tiles (its C stores overlap the next tile); below that each
  // tile is a workgroup.  Both use the split-load single-buffered schedule.
  const int64_t mt = (M + 255) / 256;
  const int64_t r256 = (mt * ((N + 255) / 256) * batch + 255) / 256;
  const int64_t r128 = (mt * ((N + 127) / 128) * batch + 255) / 256;
  if (r128 * 57 < r256 * 100) return 1;
  return r256 >= 4 ? 0 : 2;
}

// Columns [0, nm) as whole rounds of 256 x 256 tiles and the rest as 256 x
// 128 tiles in a second launch, when that costs fewer rounds than either
// tile size alone (a last round of big tiles that would run partly empty):
// returns nm, or 0 for one launch.  Costs as in gemm_lds_config.  Not from
// four rounds on, where the persistent kernel spreads a partial last round
// over its workgroups (7B-class gate projection, 21.5 rounds: the split was
// 0.6 % slower; 11008 x 4096 at T = 2048, 1.34 rounds: 238 -> 215 us).
int64_t gemm_lds_split(int64_t M, int64_t N, int64_t batch) {
  const int64_t per = ((M + 255) / 256) * batch;  // 256 x 256 tiles per column
  const int64_t nt = (N + 255) / 256;
  if ((per * nt + 255) / 256 >= 4) return 0;
  const int64_t step = 256 / std::gcd(per, (int64_t)256);
  const int64_t ntm = nt / step * step;
  if (ntm == 0 || ntm == nt) return 0;
  const int64_t r_main = per * ntm / 256;
  const int64_t n_tail = N - ntm * 256;
  const int64_t r_tail = (((M + 255) / 256) * ((n_tail + 127) / 128) * batch + 255) / 256;
  const int64_t r256 = (per * nt + 255) / 256;
  const int64_t r128 = (((M + 255) / 256) * ((N + 127) / 128) * batch + 255) / 256;
  const int64_t best = std::min(r256 * 100, r128 * 57);
  return r_main * 100 + r_tail * 57 < best ? ntm * 256 : 0;
}

hipError_t launch_gemm_lds(const GemmArgs& a, const Launch& L) {
  if (a.M <= 0 || a.N_store <= 0) return hipSuccess;
  if (a.K1 <= 0 || !a.C || a.nsplit > 1) return hipErrorInvalidValue;
  // tiled B: 32-bit offsets inside one 256-row block of k-tiles
  if (a.b1_tiled && (a.K1 + 63) / 64 * kWtRows * kWtCols * 2 >= (int64_t)kOutOfRange)
    return hipErrorInvalidValue;
  const int64_t nm = gemm_lds_split(a.M, a.N_store, a.batch > 1 ? a.batch : 1);
  if (nm > 0) {
    // the same MFMAs in the same order per output with either tile size:
    // the result does not depend on the split
    GemmArgs m = a, t = a;
    m.N_store = nm;
    m.N = std::min(a.N, nm);
    t.N_store = a.N_store - nm;
    t.N = std::max((int64_t)0, a.N - nm);
    t.C = a.C + nm;
    t.B1 = a.b1_tiled ? a.B1 + (nm / kWtRows) * ((a.K1 + 63) / 64) * (kWtRows * kWtCols)
                      : a.B1 + nm * a.ldb1;
    if (a.B2) t.B2 = a.B2 + nm * a.ldb2;
    // (timing events: the first launch's start, the second's end)
    const Launch Lm{L.s, L.e0, nullptr}, Lt{L.s, nullptr, L.e1};
    const hipError_t e = launch_gemm_lds(m, Lm);
    if (e != hipSuccess) return e;
    return launch_t<2, 2, 4, 2, 3, kDoubleBuf>(t, Lt);
  }
  switch (gemm_lds_config(a.M, a.N_store, a.batch > 1 ? a.batch : 1)) {
    case 0:  // 256 x 256, 8 waves, 2 stages, persistent
      return launch_tp<4, 2, 2, 4, 2, kSingleBufSplit>(a, L);
    case 2:
      return launch_t<4, 2, 2, 4, 2, kSingleBufSplit>(a, L);
    default:  // 256 x 128, 8 waves, 3 stages
      return launch_t<2, 2, 4, 2, 3, kDoubleBuf>(a, L);
  }
}

}  // namespace ttq
