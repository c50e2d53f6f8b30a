// Host side of the TTQ linear projection library: argument validation,
// path selection, workspace layout and kernel dispatch.  Everything here is
// plain host code; the arithmetic of the method runs in the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/ttq.h"
#include "ttq_internal.h"

using namespace ttq;

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxD = int64_t(1) << 20;
constexpr int64_t kMaxDout = int64_t(1) << 22;
constexpr int64_t kMaxT = int64_t(1) << 22;
constexpr int64_t kMaxR = 4096;
constexpr int64_t kMaxElems = int64_t(1) << 34;
// two-phase path: workspace for the dequantized weights of several requests
constexpr int64_t kMaxWhatBytes = int64_t(4) << 30;
constexpr int kFusedMaxT = 128;
// one token tile per weight tile: the GEMM quantizes its weight tiles itself
// instead of a quantize pass writing W_hat (with two token tiles the tile
// would be quantized twice, which costs as much as the pass it replaces)
constexpr int64_t kGemmQMaxT = 256;

constexpr size_t kGemvLdsMax = 128 * 1024;

// the fused kernel takes two row blocks per workgroup from this many
// workgroups on (the chip's compute units)
constexpr int64_t kFusedPairWgs = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr uint32_t known_flags() {
  return TTQ_FLAG_FORCE_FUSED | TTQ_FLAG_FORCE_TWO_PHASE;
}

struct Plan {
  int path = 0;          // 0 fused, 1 two-phase, 2 single launch (T = 1),
                         // 3 two-phase with quantization inside the GEMM
  int ntb = 1;           // fused: 16-token blocks (power of two)
  int G = 0;             // groups per row
  int frb = 1;           // fused: 16-row blocks per workgroup
  int64_t rowblocks = 0;
  int sz_ntb = 0;         // large T: 64-token blocks per request,
  int sz_csplit = 1;      // channel ranges per block,
  int sz_cps = 0;         // 512-channel chunks per range
  bool z_fused = false;   // Z = X A^T computed by the statistics pass
  int64_t rp = 0;        // rank padded to a multiple of 32
  int64_t rchunk = 1;    // two-phase: requests quantized per pass
  int zsplit = 1;        // two-phase: K splits of Z = X A^T
  int64_t zksplit = 0;   // channels per split
  size_t off_dh = 0, off_dhi = 0, off_xs = 0, off_sx = 0, off_z = 0,
         off_statp = 0, off_what = 0, off_zpart = 0;
  size_t off_zsmall = 0;  // fp32 partials of the small-M Z kernel
  size_t off_xsc = 0;     // fused, T <= 16: inverse fp16 scales of x'
  size_t total = 0;
};

bool finite_nonneg(double v) { return std::isfinite(v) && v >= 0.0; }

int validate_params(const ttq_params* prm, int64_t R) {
  if (!prm) return TTQ_ENULL;
  if (R < 0 || R > kMaxR) return TTQ_EINVAL;
  if (prm->d < 1 || prm->d > kMaxD) return TTQ_EINVAL;
  if (prm->d_out < 0 || prm->d_out > kMaxDout) return TTQ_EINVAL;
  if (prm->T < 0 || prm->T > kMaxT) return TTQ_EINVAL;
  if (prm->rank < 0) return TTQ_EINVAL;
  if (prm->bits < 1 || prm->bits > 8) return TTQ_EINVAL;
  if (prm->qformat > TTQ_QF_FP8) return TTQ_EINVAL;
  if (prm->qformat == TTQ_QF_SYM && prm->bits < 2) return TTQ_EINVAL;
  if (prm->qformat == TTQ_QF_FP8 && prm->bits != 8) return TTQ_EINVAL;
  if (prm->group <= 0 || prm->d % prm->group != 0) return TTQ_EINVAL;
  if (!(std::isfinite(prm->p) && prm->p > 0.0)) return TTQ_EINVAL;
  if (!finite_nonneg(prm->lambda) || !finite_nonneg(prm->alpha))
    return TTQ_EINVAL;
  const uint32_t known = TTQ_FLAG_FORCE_FUSED | TTQ_FLAG_FORCE_TWO_PHASE;
  if (prm->flags & ~known) return TTQ_EINVAL;
  if ((prm->flags & known) == known) return TTQ_EINVAL;
  if (prm->d * prm->d_out > kMaxElems) return TTQ_EINVAL;
  if (R * prm->T * prm->d > kMaxElems) return TTQ_EINVAL;
  if (R * prm->T * prm->d_out > kMaxElems) return TTQ_EINVAL;
  if (prm->group != 32 && prm->group != 64 && prm->group != 128 &&
      prm->group != 256)
    return TTQ_EUNSUPPORTED;
  if (prm->rank > 0 && (prm->rank % 8 != 0 || prm->rank > 1024))
    return TTQ_EUNSUPPORTED;
  if ((prm->flags & TTQ_FLAG_FORCE_FUSED) && prm->T > kFusedMaxT)
    return TTQ_EUNSUPPORTED;
  return TTQ_OK;
}

// Large T: one workgroup per 64-token block of a request; when that gives
// fewer than 256 workgroups (one per CU: the kernel holds 128 KiB of LDS)
// the channels are split into ranges of whole 512-channel chunks as well
// (the low-rank product of each range is then a float32 partial, summed in
// range order).  One round of workgroups with more chunks each beats two
// rounds (11008 -> 4096 at T = 2048: 352 -> 256 workgroups, 35 -> 25 us).
template <class Take>
void plan_stats_z(Plan& P, int64_t R, int64_t T, int64_t d, bool with_z,
                  Take& take) {
  P.sz_ntb = (int)((T + 63) / 64);
  const int64_t nck = (d + 511) / 512;
  const int64_t blocks = R * P.sz_ntb;
  int64_t cs = blocks > 0 ? (256 + blocks - 1) / blocks : 1;
  if (cs > nck) cs = nck;
  if (cs < 1) cs = 1;
  P.sz_cps = (int)((nck + cs - 1) / cs);
  P.sz_csplit = P.sz_cps > 0 ? (int)((nck + P.sz_cps - 1) / P.sz_cps) : 1;
  P.off_statp = take(sizeof(double) * R * P.sz_ntb * d);
  P.z_fused = with_z;
  if (with_z && P.sz_csplit > 1)
    P.off_zpart = take(sizeof(float) * P.sz_csplit * R * T * P.rp);
}

// the statistics pass computes Z itself for ranks up to 128 with p in {1, 2}
// (registers: larger ranks or the general-p power use the GEMM for Z; at
// rank 128 a few bytes spill, and the pass still costs less than the Z GEMM
// and its reduction: 70B-class up projection, T = 512, 30 -> 17.5 us)
bool z_in_stats(int64_t rp, double p) { return rp > 0 && rp <= 128 && (p == 2.0 || p == 1.0); }

// Z = X A^T has few output tiles (rank columns): split the channels so that
// about 512 workgroups run, each over at least 256 channels.
template <class Take>
void plan_z_split(Plan& P, int64_t M, int64_t d, Take& take) {
  const int64_t tiles = ((M + 127) / 128) * ((P.rp + 127) / 128);
  const int64_t nk = (d + 63) / 64;
  int64_t S = (512 + tiles - 1) / tiles;
  if (S > nk / 4) S = nk / 4;
  if (S < 1) S = 1;
  P.zksplit = (nk + S - 1) / S * 64;
  P.zsplit = (int)((d + P.zksplit - 1) / P.zksplit);
  if (P.zsplit > 1) P.off_zpart = take(sizeof(float) * P.zsplit * M * P.rp);
}

// Fused path, 17 to 128 tokens: every workgroup re-reads the request's whole
// x' from L2, T/16 times the bytes of its weight rows, and with several
// workgroups per CU that L2 -> CU traffic bounds the kernel.  Two row blocks
// per workgroup halve it, as long as that still gives every compute unit a
// workgroup (8 requests x 4096 rows: -18 % at T = 64, -32 % at T = 128).  At
// T <= 16 the kernel is bound by its vector ALU work instead, and the larger
// register set of two row blocks costs more than the traffic it saves.
void fused_shape(Plan& P, int64_t R, int group) {
  P.frb = 1;
  if (P.ntb >= 2 && group <= 128 && R * ((P.rowblocks + 1) / 2) >= kFusedPairWgs)
    P.frb = 2;
}

// The small-T statistics kernel writes the low-rank partials itself (its
// workgroups own 128-channel blocks) when 128-channel slices are not capped
// by the partials' size; otherwise the small-M kernel writes 256-channel ones.
bool z_parts_in_stats(int64_t rp, int64_t M, int64_t d) {
  return rp > 0 && M > 0 && lowrank_z_splits(M, d, (int)rp, 128) == (d + 127) / 128;
}

size_t z_small_bytes(int64_t rp, int64_t M, int64_t d) {
  const size_t b = lowrank_z_part_bytes(M, d, (int)rp, 256);
  const size_t f = z_parts_in_stats(rp, M, d) ? lowrank_z_part_bytes(M, d, (int)rp, 128) : 0;
  return b > f ? b : f;
}

Plan make_plan(const ttq_params* prm, int64_t R) {
  Plan P;
  const int64_t d = prm->d, dout = prm->d_out, T = prm->T;
  P.G = (int)(d / prm->group);
  P.rp = prm->rank > 0 ? (prm->rank + 31) / 32 * 32 : 0;
  bool fused = T <= kFusedMaxT;
  if (prm->flags & TTQ_FLAG_FORCE_FUSED) fused = true;
  if (prm->flags & TTQ_FLAG_FORCE_TWO_PHASE) fused = false;
  P.path = fused ? 0 : 1;
  const bool gemv_fits = d <= kGemvMaxD && gemv_lds_bytes(d, P.G) <= kGemvLdsMax;
  if (T == 1 && gemv_fits && !(prm->flags & known_flags())) P.path = 2;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  P.off_dh = take(sizeof(float) * R * d);
  P.off_dhi = take(sizeof(float) * R * d);
  if (P.rp > 0) P.off_z = take(sizeof(uint16_t) * R * T * P.rp);
  if (P.rp > 0 && T > 0 && (P.path == 2 || fused))
    P.off_zsmall = take(z_small_bytes(P.rp, R * T, d));

  if (P.path == 2) {
    P.rowblocks = (dout + 15) / 16;
  } else if (fused) {
    P.ntb = 1;
    while (P.ntb * 16 < T) P.ntb *= 2;
    P.rowblocks = (dout + 15) / 16;
    // one activation plane: bf16 for T > 16, scaled fp16 for T <= 16 (with
    // an inverse scale per group and token)
    P.off_xs = take(sizeof(uint16_t) * R * 16 * P.ntb * d);
    P.off_sx = take(sizeof(float) * R * P.G * 16 * P.ntb);
    if (T <= 16) P.off_xsc = take(sizeof(float) * R * P.G * 16 * P.ntb);
    fused_shape(P, R, prm->group);
  } else {
    const bool zf = T > 0 && z_in_stats(P.rp, prm->p);
    plan_stats_z(P, R, T, d, zf, take);
    if (P.rp > 0 && T > 0 && !zf) plan_z_split(P, R * T, d, take);
    if (T <= kGemmQMaxT && gemm_q_supported(d, prm->group, 0) &&
        !(prm->flags & TTQ_FLAG_FORCE_TWO_PHASE)) {
      // no W_hat: the GEMM quantizes its weight tiles itself (exports, when
      // asked for, come from a quantize pass that writes only them)
      P.path = 3;
    } else {
      // W_hat of up to rchunk requests at a time (at most kMaxWhatBytes)
      const int64_t per = (int64_t)sizeof(uint16_t) * what_tiled_elems(dout, d);
      P.rchunk = per > 0 ? kMaxWhatBytes / per : R;
      if (P.rchunk < 1) P.rchunk = 1;
      if (P.rchunk > R) P.rchunk = R;
      P.off_what = take((size_t)(per * P.rchunk));
    }
  }
  P.total = off;
  return P;
}

bool misaligned(const void* p, size_t a) {
  return p && (reinterpret_cast<uintptr_t>(p) % a) != 0;
}

// ---------------------------------------------------------------- timing
struct TimingState {
  bool enabled = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[K_NUM_KINDS];
  std::vector<hipEvent_t> pool;
  double total_ms[K_NUM_KINDS] = {};
  int64_t launches[K_NUM_KINDS] = {};
};
TimingState g_timing;

const char* kKernelNames[K_NUM_KINDS] = {
    "stats_small", "stats_z", "stats_final", "fused_qdq_mfma",
    "quant_what", "gemm_mfma", "lowrank_z", "gemv_t1", "splitk_reduce",
    "qgemv", "dequant", "qfused", "lowrank_zsum", "gemm_quant", "seg_copy",
    "pca_skinny", "pca_psum", "pca_chol", "pca_trsm", "pca_residual",
    "pca_complete", "stream_read"};

hipEvent_t take_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch one kernel through `launch(L)`; with timing enabled the runtime
// stamps the kernel's own start and end into a pair of events.
template <class F>
int run(KernelKind kind, hipStream_t s, F&& launch) {
  Launch L{s, nullptr, nullptr};
  if (g_timing.enabled) {
    L.e0 = take_event();
    L.e1 = take_event();
    if (!L.e0 || !L.e1) {
      if (L.e0) g_timing.pool.push_back(L.e0);
      if (L.e1) g_timing.pool.push_back(L.e1);
      L.e0 = L.e1 = nullptr;
    }
  }
  const hipError_t err = launch(L);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    if (L.e0) g_timing.pool.push_back(L.e0);
    if (L.e1) g_timing.pool.push_back(L.e1);
    return TTQ_EHIP;
  }
  if (L.e0) g_timing.pending[kind].push_back({L.e0, L.e1});
  return TTQ_OK;
}

// Failure injection for the error-path tests: with TTQ_INJECT_HIP_ERROR=1 a
// call that passed validation reports a failed launch and enqueues nothing.
bool inject_hip_error() {
  const char* inj = std::getenv("TTQ_INJECT_HIP_ERROR");
  if (inj && inj[0] == '1') {
    g_last_hip_error = (int)hipErrorLaunchFailure;
    return true;
  }
  return false;
}

// Z = X A^T (M rows) with the MFMA GEMM, split over the channels as planned
// (fp32 partials summed in split order, then rounded to bf16).
int enqueue_z_gemm(const Plan& P, char* ws, const bf16_t* Xb,
                   const bf16_t* Ab, int64_t M, int64_t d, int64_t rank,
                   bf16_t* Zb, hipStream_t s) {
  GemmArgs za{};
  za.A1 = Xb; za.lda1 = d; za.B1 = Ab; za.ldb1 = d; za.K1 = d;
  za.M = M; za.N = rank; za.N_store = P.rp;
  za.ldc = P.rp;
  if (P.zsplit > 1) {
    za.C = reinterpret_cast<float*>(ws + P.off_zpart);
    za.ksplit = P.zksplit;
    za.nsplit = P.zsplit;
    za.split_stride = M * P.rp;
  } else {
    za.Cb = Zb;
  }
  int st = run(K_LOWRANK_Z, s, [&](const Launch& L) { return launch_gemm(za, L); });
  if (st != TTQ_OK || P.zsplit <= 1) return st;
  SplitReduceArgs ra{za.C, P.zsplit, M * P.rp, Zb};
  return run(K_SPLITK_REDUCE, s, [&](const Launch& L) { return launch_splitk_reduce(ra, L); });
}

// Z = X A^T for small M (one-token, fused and packed-code routes): channel
// slices on the matrix cores, then their ordered sum.
int enqueue_z_small(const Plan& P, char* ws, const bf16_t* Xb,
                    const bf16_t* Ab, int64_t M, int64_t d, int64_t rank,
                    bf16_t* Zb, hipStream_t s, bool parts_written = false) {
  LowRankZArgs za{Xb, Ab, M, d, (int)rank, (int)P.rp, Zb,
                  reinterpret_cast<float*>(ws + P.off_zsmall)};
  if (!parts_written) {
    const int st = run(K_LOWRANK_Z, s, [&](const Launch& L) { return launch_lowrank_z_small(za, L); });
    if (st != TTQ_OK) return st;
  }
  const int ns = parts_written ? (int)((d + 127) / 128)
                               : lowrank_z_splits(M, d, (int)P.rp, 256);
  return run(K_LOWRANK_ZSUM, s, [&](const Launch& L) { return launch_lowrank_z_sum(za, ns, L); });
}

// Statistics of a large-T call (and Z = X A^T when the plan fuses it): the
// block partials, then D^{+-1/2}; with several channel ranges Z is summed
// from their float32 partials in range order.
int enqueue_stats_z(const Plan& P, char* ws, const bf16_t* Xb,
                    const bf16_t* Ab, int64_t R, int64_t T, int64_t d,
                    int64_t rank, bf16_t* Zb, int pmode, double p, double lam,
                    double alpha, float* dh, float* dhi, float* dh_export,
                    hipStream_t s) {
  const bool zf = P.z_fused && Ab && T > 0;
  StatsZArgs za{};
  za.X = Xb; za.T = T; za.d = d; za.pmode = pmode; za.p = p;
  za.ntb = P.sz_ntb; za.csplit = P.sz_csplit; za.cps = P.sz_cps;
  za.partial = reinterpret_cast<double*>(ws + P.off_statp);
  if (zf) {
    za.A = Ab; za.rank = (int)rank; za.rp = (int)P.rp;
    za.Z = Zb;
    za.Zpart = P.sz_csplit > 1 ? reinterpret_cast<float*>(ws + P.off_zpart) : nullptr;
    za.zslice = R * T * P.rp;
  }
  int st = run(K_STATS_Z, s, [&](const Launch& L) { return launch_stats_z(za, (int)R, L); });
  if (st != TTQ_OK) return st;
  StatsFinalArgs fa{};
  fa.partial = za.partial; fa.d = d; fa.nb = P.sz_ntb; fa.pmode = pmode;
  fa.p = p; fa.lam = lam; fa.alpha = alpha;
  fa.dh = dh; fa.dhi = dhi; fa.dh_export = dh_export;
  if (zf && P.sz_csplit > 1) {
    // Z summed from the channel ranges' partials in the same launch
    fa.zpart = za.Zpart; fa.zsplit = P.sz_csplit; fa.zn = za.zslice; fa.Z = Zb;
  }
  return run(K_STATS_FINAL, s, [&](const Launch& L) { return launch_stats_final(fa, (int)R, L); });
}

int linear_impl(const ttq_params* prm, int64_t R, const void* W,
                const void* X, const void* B, const void* A, float* Y,
                uint8_t* codes_out, float* scales_out, float* mins_out,
                float* dhalf_out, void* workspace, size_t workspace_bytes,
                void* stream) {
  int st = validate_params(prm, R);
  if (st != TTQ_OK) return st;
  const int64_t d = prm->d, dout = prm->d_out, T = prm->T, rank = prm->rank;
  if (R == 0) return TTQ_OK;
  if (dout > 0 && !W) return TTQ_ENULL;
  if (T > 0 && !X) return TTQ_ENULL;
  if (T > 0 && dout > 0 && !Y) return TTQ_ENULL;
  if (rank > 0 && (!B || !A)) return TTQ_ENULL;
  if ((scales_out == nullptr) != (mins_out == nullptr)) return TTQ_EINVAL;
  if (misaligned(W, 16) || misaligned(X, 16) || misaligned(B, 16) ||
      misaligned(A, 16) || misaligned(Y, 4) || misaligned(codes_out, 8) ||
      misaligned(scales_out, 4) || misaligned(mins_out, 4) ||
      misaligned(dhalf_out, 4) || misaligned(workspace, 256))
    return TTQ_EALIGN;
  const Plan P = make_plan(prm, R);
  if (P.total > 0 && !workspace) return TTQ_ENULL;
  if (workspace_bytes < P.total) return TTQ_EWORKSPACE;
  if (inject_hip_error()) return TTQ_EHIP;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* dh = reinterpret_cast<float*>(ws + P.off_dh);
  float* dhi = reinterpret_cast<float*>(ws + P.off_dhi);
  bf16_t* Zb = P.rp > 0 ? reinterpret_cast<bf16_t*>(ws + P.off_z) : nullptr;
  const bf16_t* Wb = static_cast<const bf16_t*>(W);
  const bf16_t* Xb = static_cast<const bf16_t*>(X);
  const bf16_t* Bb = static_cast<const bf16_t*>(B);
  const bf16_t* Ab = static_cast<const bf16_t*>(A);
  const int pmode = prm->p == 2.0 ? 2 : (prm->p == 1.0 ? 1 : 0);
  const float Nf = (float)((1 << prm->bits) - 1);
  const bool need_quant = dout > 0;

  if (P.path == 2) {
    if (P.rp > 0) {
      st = enqueue_z_small(P, ws, Xb, Ab, R, d, rank, Zb, s);
      if (st != TTQ_OK) return st;
    }
    GemvArgs va{};
    va.W = Wb; va.X = Xb; va.d = d; va.d_out = dout; va.G = P.G; va.Nf = Nf;
    va.pmode = pmode; va.p = prm->p; va.lam = prm->lambda; va.alpha = prm->alpha;
    va.Z = Zb; va.Blr = Bb; va.rank = (int)rank; va.rp = (int)P.rp;
    va.Y = Y; va.rowblocks = P.rowblocks; va.R = (int)R;
    va.codes_out = codes_out; va.s_out = scales_out; va.m_out = mins_out;
    va.dh_export = dhalf_out;
    va.qf = (int)prm->qformat;
    if (dout == 0) {  // statistics only: the gemv kernel needs a row block
      StatsSmallArgs sa{};
      sa.X = Xb; sa.T = T; sa.d = d; sa.pmode = pmode;
      sa.p = prm->p; sa.lam = prm->lambda; sa.alpha = prm->alpha;
      sa.dh = dh; sa.dhi = dhi; sa.dh_export = dhalf_out; sa.group = prm->group;
      return run(K_STATS_SMALL, s, [&](const Launch& L) { return launch_stats_small(sa, (int)R, L); });
    }
    return run(K_GEMV, s, [&](const Launch& L) { return launch_gemv(va, prm->group, L); });
  }
  if (P.path == 0) {
    StatsSmallArgs sa{};
    sa.X = Xb; sa.T = T; sa.d = d; sa.pmode = pmode;
    sa.p = prm->p; sa.lam = prm->lambda; sa.alpha = prm->alpha;
    sa.dh = dh; sa.dhi = dhi; sa.dh_export = dhalf_out;
    sa.xs = need_quant ? reinterpret_cast<bf16_t*>(ws + P.off_xs) : nullptr;
    sa.sx = need_quant ? reinterpret_cast<float*>(ws + P.off_sx) : nullptr;
    sa.xsc = need_quant && P.ntb == 1 ? reinterpret_cast<float*>(ws + P.off_xsc) : nullptr;
    sa.group = prm->group;
    sa.Tp = 16 * P.ntb;
    const bool zin = need_quant && z_parts_in_stats(P.rp, R * T, d);
    if (zin) {
      sa.zA = Ab; sa.zrank = (int)rank; sa.zrp = (int)P.rp;
      sa.zpart = reinterpret_cast<float*>(ws + P.off_zsmall);
    }
    st = run(K_STATS_SMALL, s, [&](const Launch& L) { return launch_stats_small(sa, (int)R, L); });
    if (st != TTQ_OK) return st;
    if (!need_quant) return TTQ_OK;
    if (P.rp > 0 && T > 0) {
      st = enqueue_z_small(P, ws, Xb, Ab, R * T, d, rank, Zb, s, zin);
      if (st != TTQ_OK) return st;
    }
    FusedArgs fa{};
    fa.W = Wb; fa.d = d; fa.d_out = dout; fa.T = T; fa.G = P.G; fa.Nf = Nf;
    fa.dh = dh; fa.xs = sa.xs; fa.sx = sa.sx; fa.xsc = sa.xsc;
    fa.Z = Zb; fa.Blr = Bb; fa.rank = (int)rank; fa.rp = (int)P.rp;
    fa.Y = Y;
    fa.rowblocks = P.rowblocks;
    fa.R = (int)R;
    fa.codes_out = codes_out; fa.s_out = scales_out; fa.m_out = mins_out;
    fa.qf = (int)prm->qformat;
    return run(K_FUSED, s, [&](const Launch& L) { return launch_fused(fa, P.ntb, prm->group, P.frb, L); });
  }

  // two-phase path: statistics (and Z, when fused) in one pass over X
  st = enqueue_stats_z(P, ws, Xb, need_quant ? Ab : nullptr, R, T, d, rank, Zb,
                       pmode, prm->p, prm->lambda, prm->alpha, dh, dhi,
                       dhalf_out, s);
  if (st != TTQ_OK) return st;
  if (!need_quant) return TTQ_OK;
  if (P.rp > 0 && !P.z_fused) {
    st = enqueue_z_gemm(P, ws, Xb, Ab, R * T, d, rank, Zb, s);
    if (st != TTQ_OK) return st;
  }
  if (P.path == 3) {
    if (codes_out || scales_out) {
      // the exports of every request, without W_hat
      QuantArgs ea{};
      ea.W = Wb; ea.d = d; ea.d_out = dout; ea.G = P.G; ea.R = (int)R; ea.Nf = Nf;
      ea.dh = dh; ea.dhi = dhi; ea.What = nullptr;
      ea.codes_out = codes_out; ea.s_out = scales_out; ea.m_out = mins_out;
      ea.qf = (int)prm->qformat;
      st = run(K_QUANT, s, [&](const Launch& L) { return launch_quant(ea, prm->group, L); });
      if (st != TTQ_OK) return st;
    }
    // every request in one launch, each with its own statistics
    GemmQArgs qa{};
    qa.X = Xb; qa.ldx = d; qa.W = Wb; qa.ldw = d;
    qa.dh = dh; qa.dhi = dhi; qa.Nf = Nf; qa.K1 = d;
    if (P.rp > 0) {
      qa.A2 = Zb; qa.lda2 = P.rp; qa.B2 = Bb; qa.ldb2 = rank; qa.K2 = rank;
    }
    qa.M = T; qa.N = dout; qa.C = Y; qa.ldc = dout;
    qa.batch = (int)R;
    qa.sX = T * d; qa.sA2 = T * P.rp; qa.sC = T * dout;
    qa.qf = (int)prm->qformat;
    return run(K_GEMM_Q, s, [&](const Launch& L) { return launch_gemm_q(qa, prm->group, 0, L); });
  }
  // requests in chunks of P.rchunk: one quantize pass (each request its own
  // W_hat), then one batched GEMM launch per chunk
  bf16_t* What = reinterpret_cast<bf16_t*>(ws + P.off_what);
  for (int64_t r0 = 0; r0 < R; r0 += P.rchunk) {
    const int64_t rc = R - r0 < P.rchunk ? R - r0 : P.rchunk;
    QuantArgs qa{};
    qa.W = Wb; qa.d = d; qa.d_out = dout; qa.G = P.G; qa.R = (int)rc; qa.Nf = Nf;
    qa.dh = dh + r0 * d; qa.dhi = dhi + r0 * d; qa.What = What;
    qa.codes_out = codes_out ? codes_out + r0 * dout * d : nullptr;
    qa.s_out = scales_out ? scales_out + r0 * dout * P.G : nullptr;
    qa.m_out = mins_out ? mins_out + r0 * dout * P.G : nullptr;
    qa.qf = (int)prm->qformat;
    st = run(K_QUANT, s, [&](const Launch& L) { return launch_quant(qa, prm->group, L); });
    if (st != TTQ_OK) return st;
    GemmArgs ga{};
    ga.A1 = Xb + r0 * T * d; ga.lda1 = d; ga.B1 = What; ga.ldb1 = d; ga.b1_tiled = 1;
    ga.K1 = d;
    if (P.rp > 0) {
      ga.A2 = Zb + r0 * T * P.rp; ga.lda2 = P.rp;
      ga.B2 = Bb; ga.ldb2 = rank; ga.K2 = rank;
    }
    ga.M = T; ga.N = dout; ga.N_store = dout;
    ga.C = Y + r0 * T * dout; ga.ldc = dout;
    ga.batch = (int)rc;
    ga.sA1 = T * d; ga.sB1 = what_tiled_elems(dout, d); ga.sA2 = T * P.rp; ga.sB2 = 0;
    ga.sC = T * dout;
    st = run(K_GEMM, s, [&](const Launch& L) { return launch_gemm_lds(ga, L); });
    if (st != TTQ_OK) return st;
  }
  return TTQ_OK;
}


// ------------------------------------------------- quantize once, decode
int container_bits(int bits) {
  return bits <= 1 ? 1 : (bits <= 2 ? 2 : (bits <= 4 ? 4 : 8));
}

int packed_row_bytes(const ttq_params* prm, int64_t* rb) {
  const int64_t rbits = prm->d * container_bits(prm->bits);
  if (rbits % 128 != 0) return TTQ_EUNSUPPORTED;
  *rb = rbits / 8;
  return TTQ_OK;
}

// ttq_quantize reads neither rank nor the path flags
ttq_params quantize_view(const ttq_params* prm) {
  ttq_params q = *prm;
  q.rank = 0;
  q.flags = 0;
  return q;
}

// ttq_qmatmul reads neither the statistics constants nor FORCE_FUSED
ttq_params qmatmul_view(const ttq_params* prm) {
  ttq_params q = *prm;
  q.p = 1.0;
  q.lambda = 0.0;
  q.alpha = 0.0;
  q.flags &= TTQ_FLAG_FORCE_TWO_PHASE;
  return q;
}

int validate_packed(const ttq_params* prm, const ttq_params& q, int64_t* rb) {
  if (!prm) return TTQ_ENULL;
  if (prm->flags & ~known_flags()) return TTQ_EINVAL;
  const int st = validate_params(&q, 1);
  if (st != TTQ_OK) return st;
  return packed_row_bytes(&q, rb);
}

// path 0: one statistics kernel (T <= 128); 1: partials + final
Plan make_quantize_plan(const ttq_params& q) {
  Plan P;
  P.G = (int)(q.d / q.group);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  P.off_dh = take(sizeof(float) * q.d);
  P.path = q.T <= kFusedMaxT ? 0 : 1;
  if (P.path == 1) plan_stats_z(P, 1, q.T, q.d, false, take);
  P.total = off;
  return P;
}

// path 2: one-token contraction of the codes; 0: x' from the stored
// D^{-1/2}, then the codes on the matrix cores (T <= 128); 1: dequantize +
// MFMA GEMM
Plan make_qmatmul_plan(const ttq_params& q, int cb) {
  Plan P;
  const int64_t d = q.d, T = q.T;
  P.G = (int)(d / q.group);
  P.rp = q.rank > 0 ? (q.rank + 31) / 32 * 32 : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  if (P.rp > 0) P.off_z = take(sizeof(uint16_t) * T * P.rp);
  const bool fits = qgemv_lds_bytes(d, cb, q.group) <= kGemvLdsMax;
  const bool forced = (q.flags & TTQ_FLAG_FORCE_TWO_PHASE) != 0;
  P.path = (T == 1 && fits && !forced) ? 2 : (T <= kFusedMaxT && !forced ? 0 : 1);
  // more tokens: the GEMM expands the codes itself (no W_hat in HBM)
  if (P.path == 1 && !forced && gemm_q_supported(d, q.group, cb)) P.path = 3;
  if (P.rp > 0 && T > 0 && (P.path == 0 || P.path == 2))
    P.off_zsmall = take(z_small_bytes(P.rp, T, d));
  if (P.path == 0 && T > 0 && q.d_out > 0) {
    P.ntb = 1;
    while (P.ntb * 16 < T) P.ntb *= 2;
    // one activation plane: scaled fp16 for T <= 16 (with an inverse scale
    // per group and token), bf16 above
    P.off_xs = take(sizeof(uint16_t) * 16 * P.ntb * d);
    P.off_sx = take(sizeof(float) * P.G * 16 * P.ntb);
    if (T <= 16) P.off_xsc = take(sizeof(float) * P.G * 16 * P.ntb);
  }
  if ((P.path == 1 || P.path == 3) && T > 0 && q.d_out > 0) {
    if (P.path == 1) P.off_what = take(sizeof(uint16_t) * q.d_out * d);
    if (P.rp > 0) plan_z_split(P, T, d, take);
  }
  P.total = off;
  return P;
}

int quantize_impl(const ttq_params* prm, const void* W, const void* X,
                  uint8_t* codes, float* scales, float* mins, float* dhalf_inv,
                  float* dhalf_out, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!prm) return TTQ_ENULL;
  const ttq_params q = quantize_view(prm);
  int64_t rb = 0;
  int st = validate_packed(prm, q, &rb);
  if (st != TTQ_OK) return st;
  const int64_t d = q.d, dout = q.d_out, T = q.T;
  if (dout > 0 && (!W || !codes || !scales || !mins)) return TTQ_ENULL;
  if (T > 0 && !X) return TTQ_ENULL;
  if (!dhalf_inv) return TTQ_ENULL;
  if (misaligned(W, 16) || misaligned(X, 16) || misaligned(codes, 16) ||
      misaligned(scales, 4) || misaligned(mins, 4) ||
      misaligned(dhalf_inv, 16) || misaligned(dhalf_out, 4) ||
      misaligned(workspace, 256))
    return TTQ_EALIGN;
  const Plan P = make_quantize_plan(q);
  if (P.total > 0 && !workspace) return TTQ_ENULL;
  if (workspace_bytes < P.total) return TTQ_EWORKSPACE;
  if (inject_hip_error()) return TTQ_EHIP;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* dh = reinterpret_cast<float*>(ws + P.off_dh);
  const bf16_t* Xb = static_cast<const bf16_t*>(X);
  const int pmode = q.p == 2.0 ? 2 : (q.p == 1.0 ? 1 : 0);
  if (P.path == 0) {
    StatsSmallArgs sa{};
    sa.X = Xb; sa.T = T; sa.d = d; sa.pmode = pmode;
    sa.p = q.p; sa.lam = q.lambda; sa.alpha = q.alpha;
    sa.dh = dh; sa.dhi = dhalf_inv; sa.dh_export = dhalf_out; sa.group = q.group;
    st = run(K_STATS_SMALL, s, [&](const Launch& L) { return launch_stats_small(sa, 1, L); });
  } else {
    st = enqueue_stats_z(P, ws, Xb, nullptr, 1, T, d, 0, nullptr, pmode, q.p,
                         q.lambda, q.alpha, dh, dhalf_inv, dhalf_out, s);
  }
  if (st != TTQ_OK || dout == 0) return st;
  QuantArgs qa{};
  qa.W = static_cast<const bf16_t*>(W); qa.d = d; qa.d_out = dout; qa.G = P.G;
  qa.R = 1; qa.Nf = (float)((1 << q.bits) - 1);
  qa.dh = dh; qa.dhi = dhalf_inv;
  qa.s_out = scales; qa.m_out = mins;
  qa.packed = codes; qa.cb = container_bits(q.bits); qa.row_bytes = rb;
  qa.qf = (int)q.qformat;
  return run(K_QUANT, s, [&](const Launch& L) { return launch_quant(qa, q.group, L); });
}

int qmatmul_impl(const ttq_params* prm, const uint8_t* codes,
                 const float* scales, const float* mins,
                 const float* dhalf_inv, const void* X, const void* B,
                 const void* A, float* Y, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (!prm) return TTQ_ENULL;
  const ttq_params q = qmatmul_view(prm);
  int64_t rb = 0;
  int st = validate_packed(prm, q, &rb);
  if (st != TTQ_OK) return st;
  const int64_t d = q.d, dout = q.d_out, T = q.T, rank = q.rank;
  const int cb = container_bits(q.bits);
  if (dout > 0 && (!codes || !scales || !mins)) return TTQ_ENULL;
  if (!dhalf_inv) return TTQ_ENULL;
  if (T > 0 && !X) return TTQ_ENULL;
  if (T > 0 && dout > 0 && !Y) return TTQ_ENULL;
  if (rank > 0 && (!B || !A)) return TTQ_ENULL;
  if (misaligned(codes, 16) || misaligned(scales, 4) || misaligned(mins, 4) ||
      misaligned(dhalf_inv, 16) || misaligned(X, 16) || misaligned(B, 16) ||
      misaligned(A, 16) || misaligned(Y, 4) || misaligned(workspace, 256))
    return TTQ_EALIGN;
  const Plan P = make_qmatmul_plan(q, cb);
  if (P.total > 0 && !workspace) return TTQ_ENULL;
  if (workspace_bytes < P.total) return TTQ_EWORKSPACE;
  if (inject_hip_error()) return TTQ_EHIP;
  if (T == 0 || dout == 0) return TTQ_OK;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  bf16_t* Zb = P.rp > 0 ? reinterpret_cast<bf16_t*>(ws + P.off_z) : nullptr;
  const bf16_t* Xb = static_cast<const bf16_t*>(X);
  const bf16_t* Bb = static_cast<const bf16_t*>(B);
  const bf16_t* Ab = static_cast<const bf16_t*>(A);
  if (P.path == 2) {
    if (P.rp > 0) {
      st = enqueue_z_small(P, ws, Xb, Ab, 1, d, rank, Zb, s);
      if (st != TTQ_OK) return st;
    }
    QGemvArgs ga{};
    ga.packed = codes; ga.row_bytes = rb; ga.s = scales; ga.m = mins;
    ga.dhi = dhalf_inv; ga.X = Xb; ga.d = d; ga.d_out = dout; ga.G = P.G;
    ga.Z = Zb; ga.Blr = Bb; ga.rank = (int)rank; ga.Y = Y;
    ga.qf = (int)q.qformat;
    return run(K_QGEMV, s, [&](const Launch& L) { return launch_qgemv(ga, q.group, cb, L); });
  }
  if (P.path == 0) {
    StatsSmallArgs sa{};
    sa.X = Xb; sa.T = T; sa.d = d; sa.pmode = 2; sa.p = 2.0;
    sa.dhi_in = dhalf_inv;
    sa.quarter = 1;
    sa.xs = reinterpret_cast<bf16_t*>(ws + P.off_xs);
    sa.sx = reinterpret_cast<float*>(ws + P.off_sx);
    sa.xsc = P.ntb == 1 ? reinterpret_cast<float*>(ws + P.off_xsc) : nullptr;
    sa.group = q.group;
    sa.Tp = 16 * P.ntb;
    const bool zin = z_parts_in_stats(P.rp, T, d);
    if (zin) {
      sa.zA = Ab; sa.zrank = (int)rank; sa.zrp = (int)P.rp;
      sa.zpart = reinterpret_cast<float*>(ws + P.off_zsmall);
    }
    st = run(K_STATS_SMALL, s, [&](const Launch& L) { return launch_stats_small(sa, 1, L); });
    if (st != TTQ_OK) return st;
    if (P.rp > 0) {
      st = enqueue_z_small(P, ws, Xb, Ab, T, d, rank, Zb, s, zin);
      if (st != TTQ_OK) return st;
    }
    QFusedArgs fa{};
    fa.packed = codes; fa.row_bytes = rb; fa.s = scales; fa.m = mins;
    fa.xs = sa.xs; fa.sx = sa.sx; fa.xsc = sa.xsc;
    fa.d = d; fa.d_out = dout; fa.T = T; fa.G = P.G;
    fa.Z = Zb; fa.Blr = Bb; fa.rank = (int)rank; fa.rp = (int)P.rp;
    fa.Y = Y;
    fa.qf = (int)q.qformat;
    return run(K_QFUSED, s, [&](const Launch& L) { return launch_qfused(fa, P.ntb, q.group, cb, L); });
  }
  if (P.path == 3) {
    if (P.rp > 0) {
      st = enqueue_z_gemm(P, ws, Xb, Ab, T, d, rank, Zb, s);
      if (st != TTQ_OK) return st;
    }
    GemmQArgs qa{};
    qa.X = Xb; qa.ldx = d;
    qa.packed = codes; qa.row_bytes = rb; qa.s = scales; qa.m = mins; qa.G = P.G;
    qa.dhi = dhalf_inv; qa.K1 = d;
    if (P.rp > 0) {
      qa.A2 = Zb; qa.lda2 = P.rp; qa.B2 = Bb; qa.ldb2 = rank; qa.K2 = rank;
    }
    qa.M = T; qa.N = dout; qa.C = Y; qa.ldc = dout;
    qa.batch = 1;
    qa.qf = (int)q.qformat;
    return run(K_GEMM_Q, s, [&](const Launch& L) { return launch_gemm_q(qa, q.group, cb, L); });
  }
  bf16_t* What = reinterpret_cast<bf16_t*>(ws + P.off_what);
  DequantArgs da{};
  da.packed = codes; da.row_bytes = rb; da.s = scales; da.m = mins;
  da.dhi = dhalf_inv; da.d = d; da.d_out = dout; da.G = P.G; da.What = What;
  da.qf = (int)q.qformat;
  st = run(K_DEQUANT, s, [&](const Launch& L) { return launch_dequant(da, q.group, cb, L); });
  if (st != TTQ_OK) return st;
  if (P.rp > 0) {
    st = enqueue_z_gemm(P, ws, Xb, Ab, T, d, rank, Zb, s);
    if (st != TTQ_OK) return st;
  }
  GemmArgs ga{};
  ga.A1 = Xb; ga.lda1 = d; ga.B1 = What; ga.ldb1 = d; ga.K1 = d;
  if (P.rp > 0) {
    ga.A2 = Zb; ga.lda2 = P.rp;
    ga.B2 = Bb; ga.ldb2 = rank; ga.K2 = rank;
  }
  ga.M = T; ga.N = dout; ga.N_store = dout;
  ga.C = Y; ga.ldc = dout;
  ga.batch = 1;
  return run(K_GEMM, s, [&](const Launch& L) { return launch_gemm_lds(ga, L); });
}

// ------------------------------------------------- continuous batching
// Requests of different lengths packed in one X [sum T_r][d] (see
// k_segment.hip).  Requests of one length class are computed as one batched
// call: a class groups the lengths that run the same kernels with the same
// per-token arithmetic (1; 2..16; 17..32; 33..64; 65..128), padded with zero
// tokens to the longest request of the batch; longer requests run alone at
// their own length.  Each request's D, codes and Y rows are then those of the
// request alone.  Without exports a batch takes every request of its class;
// with exports (written in request order) only runs of consecutive requests.
int64_t seg_class(int64_t T) {
  if (T <= 1) return T;
  if (T <= 16) return 16;
  if (T <= kFusedMaxT) {
    int64_t c = 32;
    while (c < T) c *= 2;
    return c;
  }
  return -1;  // alone, at its own length
}

struct SegBatch {
  std::vector<int64_t> seg;  // requests, in request order
  int64_t Tpad = 0;
  bool direct = false;       // consecutive requests of length Tpad: no copies
  size_t ws = 0;             // workspace of the batched call
  size_t xpad = 0, ypad = 0;
};

int check_offsets(const ttq_params* prm, int64_t n_seg, const int64_t* off) {
  if (n_seg < 0 || n_seg > kMaxR * 64) return TTQ_EINVAL;
  if (n_seg > 0 && !off) return TTQ_ENULL;
  const int st = validate_params(prm, 1);
  if (st != TTQ_OK) return st;
  if (n_seg > 0 && (off[0] != 0 || off[n_seg] != prm->T)) return TTQ_EINVAL;
  for (int64_t i = 0; i < n_seg; ++i)
    if (off[i + 1] < off[i]) return TTQ_EINVAL;
  return TTQ_OK;
}

int plan_segments(const ttq_params* prm, int64_t n_seg, const int64_t* off,
                  bool by_class, std::vector<SegBatch>* out, size_t* total) {
  // a path flag: every request alone (the flag fixes its kernels)
  const bool alone = (prm->flags & known_flags()) != 0;
  auto len = [&](int64_t i) { return off[i + 1] - off[i]; };
  auto cls = [&](int64_t i) { return alone ? -1 : seg_class(len(i)); };
  std::vector<SegBatch> batches;
  std::vector<bool> taken((size_t)n_seg, false);
  for (int64_t i = 0; i < n_seg; ++i) {
    if (taken[(size_t)i]) continue;
    const int64_t c = cls(i);
    SegBatch b;
    b.seg.push_back(i);
    taken[(size_t)i] = true;
    if (c > 0) {
      for (int64_t k = i + 1; k < n_seg && (int64_t)b.seg.size() < kSegMax; ++k) {
        if (taken[(size_t)k]) continue;
        if (cls(k) != c) {
          if (by_class) continue;
          break;
        }
        b.seg.push_back(k);
        taken[(size_t)k] = true;
      }
    }
    batches.push_back(std::move(b));
  }
  size_t need = 0;
  for (SegBatch& b : batches) {
    const int64_t n = (int64_t)b.seg.size();
    b.Tpad = 0;
    for (int64_t k : b.seg) b.Tpad = std::max(b.Tpad, len(k));
    b.direct = true;
    for (int64_t j = 0; j < n; ++j)
      if (b.seg[(size_t)j] != b.seg[0] + j || len(b.seg[(size_t)j]) != b.Tpad)
        b.direct = false;
    ttq_params q = *prm;
    q.T = b.Tpad;
    const int st = validate_params(&q, n);
    if (st != TTQ_OK) return st;
    b.ws = make_plan(&q, n).total;
    if (!b.direct) {
      b.xpad = align_up(sizeof(uint16_t) * n * b.Tpad * prm->d, 256);
      b.ypad = align_up(sizeof(float) * n * b.Tpad * prm->d_out, 256);
    }
    need = std::max(need, align_up(b.ws, 256) + b.xpad + b.ypad);
  }
  if (out) *out = std::move(batches);
  *total = need;
  return TTQ_OK;
}

// workspace for either kind of call (with or without exports)
int segmented_workspace(const ttq_params* prm, int64_t n_seg,
                        const int64_t* off, size_t* total) {
  int st = check_offsets(prm, n_seg, off);
  if (st != TTQ_OK) return st;
  size_t a = 0, b = 0;
  st = plan_segments(prm, n_seg, off, true, nullptr, &a);
  if (st != TTQ_OK) return st;
  st = plan_segments(prm, n_seg, off, false, nullptr, &b);
  if (st != TTQ_OK) return st;
  *total = std::max(a, b);
  return TTQ_OK;
}

int segmented_impl(const ttq_params* prm, int64_t n_seg, const int64_t* off,
                   const void* W, const void* X, const void* B, const void* A,
                   float* Y, uint8_t* codes_out, float* scales_out,
                   float* mins_out, float* dhalf_out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  size_t need = 0;
  int st = segmented_workspace(prm, n_seg, off, &need);
  if (st != TTQ_OK) return st;
  if (n_seg == 0) return TTQ_OK;
  const int64_t d = prm->d, dout = prm->d_out, G = d / prm->group;
  if (dout > 0 && !W) return TTQ_ENULL;
  if (prm->T > 0 && !X) return TTQ_ENULL;
  if (prm->T > 0 && dout > 0 && !Y) return TTQ_ENULL;
  if ((scales_out == nullptr) != (mins_out == nullptr)) return TTQ_EINVAL;
  if (misaligned(workspace, 256)) return TTQ_EALIGN;
  if (need > 0 && !workspace) return TTQ_ENULL;
  if (workspace_bytes < need) return TTQ_EWORKSPACE;
  const bool exports = codes_out || scales_out || mins_out || dhalf_out;
  std::vector<SegBatch> batches;
  size_t unused = 0;
  st = plan_segments(prm, n_seg, off, !exports, &batches, &unused);
  if (st != TTQ_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bf16_t* Xb = static_cast<const bf16_t*>(X);
  for (const SegBatch& b : batches) {
    const int64_t n = (int64_t)b.seg.size(), s0 = b.seg[0];
    if (b.Tpad == 0 && !exports) continue;  // empty requests, nothing asked
    ttq_params q = *prm;
    q.T = b.Tpad;
    // exports only with runs of consecutive requests: slots s0 .. s0 + n - 1
    uint8_t* co = codes_out ? codes_out + s0 * dout * d : nullptr;
    float* so = scales_out ? scales_out + s0 * dout * G : nullptr;
    float* mo = mins_out ? mins_out + s0 * dout * G : nullptr;
    float* dho = dhalf_out ? dhalf_out + s0 * d : nullptr;
    void* bws = b.ws > 0 ? ws : nullptr;
    if (b.direct) {
      st = linear_impl(&q, n, W, b.Tpad > 0 ? Xb + off[s0] * d : nullptr, B, A,
                       Y ? Y + off[s0] * dout : nullptr, co, so, mo, dho, bws,
                       b.ws, stream);
      if (st != TTQ_OK) return st;
      continue;
    }
    const size_t inner = align_up(b.ws, 256);
    bf16_t* xpad = reinterpret_cast<bf16_t*>(ws + inner);
    float* ypad = reinterpret_cast<float*>(ws + inner + b.xpad);
    SegCopyArgs ca{};
    ca.n = (int)n;
    ca.Tpad = b.Tpad;
    for (int64_t k = 0; k < n; ++k) {
      ca.off[k] = off[b.seg[(size_t)k]];
      ca.len[k] = off[b.seg[(size_t)k] + 1] - off[b.seg[(size_t)k]];
    }
    ca.src = Xb;
    ca.dst = xpad;
    ca.row_bytes = d * (int64_t)sizeof(uint16_t);
    ca.scatter = 0;
    st = run(K_SEG_COPY, s, [&](const Launch& L) { return launch_seg_copy(ca, L); });
    if (st != TTQ_OK) return st;
    st = linear_impl(&q, n, W, xpad, B, A, ypad, co, so, mo, dho, bws, b.ws, stream);
    if (st != TTQ_OK) return st;
    if (dout == 0) continue;
    ca.src = ypad;
    ca.dst = Y;
    ca.row_bytes = dout * (int64_t)sizeof(float);
    ca.scatter = 1;
    st = run(K_SEG_COPY, s, [&](const Launch& L) { return launch_seg_copy(ca, L); });
    if (st != TTQ_OK) return st;
  }
  return TTQ_OK;
}

// ------------------------------------------------- low-rank factors by PCA
// (k_pca.hip).  Reads d, d_out, rank (the r of B and A), T (0: the principal
// subspace of W; > 0: of W D^{1/2}, D from X with p, lambda, alpha); bits,
// group, flags and qformat are not read.
int validate_pca(const ttq_params* prm, int32_t iters) {
  if (!prm) return TTQ_ENULL;
  if (prm->d < 1 || prm->d > kMaxD) return TTQ_EINVAL;
  if (prm->d_out < 1 || prm->d_out > kMaxDout) return TTQ_EINVAL;
  if (prm->T < 0 || prm->T > kMaxT) return TTQ_EINVAL;
  if (prm->d * prm->d_out > kMaxElems || prm->T * prm->d > kMaxElems) return TTQ_EINVAL;
  if (iters < 0 || iters > 16) return TTQ_EINVAL;
  const int64_t r = prm->rank;
  if (r < 1 || r > prm->d || r > prm->d_out) return TTQ_EINVAL;
  if (r != 8 && r != 16 && r != 32 && r != 64 && r != 128) return TTQ_EUNSUPPORTED;
  if (prm->T > 0) {
    if (prm->d % 8 != 0) return TTQ_EUNSUPPORTED;  // 16-byte token loads
    if (!(std::isfinite(prm->p) && prm->p > 0.0)) return TTQ_EINVAL;
    if (!finite_nonneg(prm->lambda) || !finite_nonneg(prm->alpha)) return TTQ_EINVAL;
  }
  return TTQ_OK;
}

struct PcaPlan {
  int sp_nt = 1, sp_tn = 1, sp_gy = 1, sp_gz = 1;  // splits of the products
  size_t off_dh = 0, off_dhi = 0, off_statp = 0, off_y = 0, off_z = 0,
         off_part = 0, off_g = 0, off_r = 0, off_def = 0;
  Plan stats;  // token slices of the norm partials (T > kFusedMaxT)
  size_t total = 0;
};

PcaPlan make_pca_plan(const ttq_params* prm) {
  PcaPlan P;
  const int64_t d = prm->d, dout = prm->d_out, n = prm->rank, T = prm->T;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  if (T > 0) {
    P.off_dh = take(sizeof(float) * d);
    P.off_dhi = take(sizeof(float) * d);
    if (T > kFusedMaxT) {
      plan_stats_z(P.stats, 1, T, d, false, take);
      P.off_statp = P.stats.off_statp;
    }
  }
  P.off_y = take(sizeof(float) * dout * n);
  P.off_z = take(sizeof(float) * d * n);
  P.sp_nt = skinny_splits(dout, d);   // Y = M Z        (rows d', K d)
  P.sp_tn = skinny_splits(d, dout);   // Z = M^T Q      (rows d, K d')
  P.sp_gy = skinny_splits(n, dout);   // Gram of Y
  P.sp_gz = skinny_splits(n, d);      // Gram of Z
  size_t part = 0;
  auto need = [&](int sp, int64_t rows) {
    const size_t b = sizeof(float) * sp * rows * n;
    if (b > part) part = b;
  };
  need(P.sp_nt, dout);
  need(P.sp_tn, d);
  need(P.sp_gy, n);
  need(P.sp_gz, n);
  need(1, dout);  // Y R^{-1} (r <= 64)
  need(1, d);
  P.off_part = take(part);
  P.off_g = take(sizeof(float) * n * n);
  P.off_r = take(sizeof(float) * n * n);
  P.off_def = take(sizeof(int) * n);
  P.total = off;
  return P;
}

int pca_impl(const ttq_params* prm, int32_t iters, const void* W,
             const void* X, const float* Omega, void* B_out, void* A_out,
             void* Wres_out, void* workspace, size_t workspace_bytes,
             void* stream) {
  int st = validate_pca(prm, iters);
  if (st != TTQ_OK) return st;
  const int64_t d = prm->d, dout = prm->d_out, n = prm->rank, T = prm->T;
  if (!W || !Omega || !B_out || !A_out) return TTQ_ENULL;
  if (T > 0 && !X) return TTQ_ENULL;
  if (misaligned(W, 16) || misaligned(X, 16) || misaligned(Omega, 16) ||
      misaligned(B_out, 16) || misaligned(A_out, 16) ||
      misaligned(Wres_out, 16) || misaligned(workspace, 256))
    return TTQ_EALIGN;
  const PcaPlan P = make_pca_plan(prm);
  if (!workspace) return TTQ_ENULL;
  if (workspace_bytes < P.total) return TTQ_EWORKSPACE;
  if (inject_hip_error()) return TTQ_EHIP;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bf16_t* Wb = static_cast<const bf16_t*>(W);
  float* Y = reinterpret_cast<float*>(ws + P.off_y);
  float* Z = reinterpret_cast<float*>(ws + P.off_z);
  float* part = reinterpret_cast<float*>(ws + P.off_part);
  float* G = reinterpret_cast<float*>(ws + P.off_g);
  float* Rf = reinterpret_cast<float*>(ws + P.off_r);
  int* defic = reinterpret_cast<int*>(ws + P.off_def);
  const float* dh = nullptr;

  if (T > 0) {  // D of the current activations, as in ttq_linear
    const bf16_t* Xb = static_cast<const bf16_t*>(X);
    float* dhw = reinterpret_cast<float*>(ws + P.off_dh);
    float* dhiw = reinterpret_cast<float*>(ws + P.off_dhi);
    const int pmode = prm->p == 2.0 ? 2 : (prm->p == 1.0 ? 1 : 0);
    if (T <= kFusedMaxT) {
      StatsSmallArgs sa{};
      sa.X = Xb; sa.T = T; sa.d = d; sa.pmode = pmode;
      sa.p = prm->p; sa.lam = prm->lambda; sa.alpha = prm->alpha;
      sa.dh = dhw; sa.dhi = dhiw; sa.group = 32;
      st = run(K_STATS_SMALL, s, [&](const Launch& L) { return launch_stats_small(sa, 1, L); });
    } else {
      Plan sp = P.stats;
      sp.off_statp = P.off_statp;
      st = enqueue_stats_z(sp, ws, Xb, nullptr, 1, T, d, 0, nullptr, pmode,
                           prm->p, prm->lambda, prm->alpha, dhw, dhiw, nullptr, s);
    }
    if (st != TTQ_OK) return st;
    dh = dhw;
  }

  // C[rows][n] = (A_s or A_s^T) Bm through the split partials
  auto product = [&](bool tn, bool a_bf16, const void* A, int64_t lda,
                     const float* scale, int64_t rows, int64_t K,
                     const float* Bm, int splits, float* out, bf16_t* out_b,
                     bf16_t* out_bt) -> int {
    SkinnyArgs ka{};
    ka.A = A; ka.lda = lda; ka.scale = scale; ka.Bm = Bm; ka.ldb = n;
    ka.rows = rows; ka.K = K; ka.n = (int)n; ka.kc = skinny_kc(K, splits);
    ka.part = part;
    int r = run(K_SKINNY, s, [&](const Launch& L) { return launch_skinny(ka, tn, a_bf16, L); });
    if (r != TTQ_OK) return r;
    PsumArgs pa{};
    pa.part = part; pa.nsplit = (int)((K + ka.kc - 1) / ka.kc);
    pa.rows = rows; pa.n = n; pa.out = out; pa.out_bf16 = out_b; pa.out_bf16_t = out_bt;
    return run(K_PSUM, s, [&](const Launch& L) { return launch_psum(pa, L); });
  };
  // CholeskyQR of the float32 panel V [m][n], in place: two passes for the
  // final basis (CholeskyQR2), one for the intermediate panels of the power
  // iteration, which only carry the subspace to the next product.  Between
  // the two passes of the final basis, columns whose pivot was dropped (a
  // panel of rank below n) are replaced by pseudo-random columns, so the
  // second pass returns n orthonormal columns in every case.
  auto orth = [&](float* V, int64_t m, int sp_gram, int passes) -> int {
    for (int pass = 0; pass < passes; ++pass) {
      int* df = passes == 2 && pass == 0 ? defic : nullptr;
      int r = product(true, false, V, n, nullptr, n, m, V, sp_gram, G, nullptr, nullptr);
      if (r != TTQ_OK) return r;
      if (n <= 64) {  // R^{-1} in one wave, then V R^{-1} as a product
        r = run(K_CHOL, s, [&](const Launch& L) { return launch_cholinv(G, Rf, (int)n, df, L); });
        if (r != TTQ_OK) return r;
        r = product(false, false, V, n, nullptr, m, n, Rf, 1, V, nullptr, nullptr);
      } else {
        r = run(K_CHOL, s, [&](const Launch& L) { return launch_chol(G, Rf, (int)n, df, L); });
        if (r != TTQ_OK) return r;
        r = run(K_TRSM, s, [&](const Launch& L) { return launch_trsm(V, Rf, m, (int)n, L); });
      }
      if (r != TTQ_OK) return r;
      if (df)
        r = run(K_PCA_COMPLETE, s, [&](const Launch& L) { return launch_pca_complete(V, m, (int)n, df, L); });
      if (r != TTQ_OK) return r;
    }
    return TTQ_OK;
  };

  // Q = orth(M Omega)
  st = product(false, true, Wb, d, dh, dout, d, Omega, P.sp_nt, Y, nullptr, nullptr);
  if (st == TTQ_OK) st = orth(Y, dout, P.sp_gy, iters == 0 ? 2 : 1);
  for (int it = 0; it < iters && st == TTQ_OK; ++it) {
    // Z = orth(M^T Q) = orth(D^{1/2} W^T Q);  Q = orth(M Z)
    st = product(true, true, Wb, d, dh, d, dout, Y, P.sp_tn, Z, nullptr, nullptr);
    if (st == TTQ_OK) st = orth(Z, d, P.sp_gz, 1);
    if (st == TTQ_OK)
      st = product(false, true, Wb, d, dh, dout, d, Z, P.sp_nt, Y, nullptr, nullptr);
    if (st == TTQ_OK) st = orth(Y, dout, P.sp_gy, it + 1 == iters ? 2 : 1);
  }
  if (st != TTQ_OK) return st;
  // B = bf16(Q); A = bf16(Q^T W), written transposed from W^T Q
  bf16_t* Bb = static_cast<bf16_t*>(B_out);
  bf16_t* Ab = static_cast<bf16_t*>(A_out);
  {
    PsumArgs pa{};
    pa.part = Y; pa.nsplit = 1; pa.rows = dout; pa.n = n; pa.out_bf16 = Bb;
    st = run(K_PSUM, s, [&](const Launch& L) { return launch_psum(pa, L); });
    if (st != TTQ_OK) return st;
  }
  st = product(true, true, Wb, d, nullptr, d, dout, Y, P.sp_tn, Z, nullptr, Ab);
  if (st != TTQ_OK || !Wres_out) return st;
  LrResidualArgs ra{};
  ra.W = Wb; ra.B = Bb; ra.A = Ab; ra.Wres = static_cast<bf16_t*>(Wres_out);
  ra.d = d; ra.d_out = dout;
  return run(K_LR_RESIDUAL, s, [&](const Launch& L) { return launch_lr_residual(ra, (int)n, L); });
}

// ------------------------------------------- allocation-free entry point
// Scratch for callers that cannot allocate: one array per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in symbol): its device address is looked up once
// per device with that device current, and that pointer is what the kernels
// receive.  Calls that overlap on one GPU share the array and race.
constexpr size_t kScratchBytes = TTQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// device address of this device's scratch array (looked up on first use)
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return TTQ_EHIP;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return TTQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return TTQ_EHIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TTQ_OK;
}

}  // namespace

extern "C" {

int ttq_linear_noalloc(const ttq_params* prm, int64_t n_requests,
                       const void* W, const void* X, const void* B,
                       const void* A, float* Y, uint8_t* codes_out,
                       float* scales_out, float* mins_out, float* dhalf_out,
                       void* stream) {
  // the plan's size is checked on the host before anything touches HIP
  int st = validate_params(prm, n_requests);
  if (st != TTQ_OK) return st;
  if (n_requests == 0) return TTQ_OK;
  const size_t need = make_plan(prm, n_requests).total;
  if (need > kScratchBytes) return TTQ_EWORKSPACE;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != TTQ_OK) return st;
  return linear_impl(prm, n_requests, W, X, B, A, Y, codes_out, scales_out,
                     mins_out, dhalf_out, ws, kScratchBytes, stream);
}

int ttq_workspace_bytes(const ttq_params* prm, int64_t n_requests,
                        size_t* bytes) {
  if (!bytes) return TTQ_ENULL;
  const int st = validate_params(prm, n_requests);
  if (st != TTQ_OK) return st;
  *bytes = n_requests == 0 ? 0 : make_plan(prm, n_requests).total;
  return TTQ_OK;
}

int ttq_linear(const ttq_params* prm, const void* W, const void* X,
               const void* B, const void* A, float* Y, uint8_t* codes_out,
               float* scales_out, float* mins_out, float* dhalf_out,
               void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl(prm, 1, W, X, B, A, Y, codes_out, scales_out, mins_out,
                     dhalf_out, workspace, workspace_bytes, stream);
}

int ttq_linear_batched(const ttq_params* prm, int64_t n_requests,
                       const void* W, const void* X, const void* B,
                       const void* A, float* Y, uint8_t* codes_out,
                       float* scales_out, float* mins_out, float* dhalf_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl(prm, n_requests, W, X, B, A, Y, codes_out, scales_out,
                     mins_out, dhalf_out, workspace, workspace_bytes, stream);
}

int ttq_segmented_workspace_bytes(const ttq_params* prm, int64_t n_segments,
                                  const int64_t* seg_offsets, size_t* bytes) {
  if (!bytes) return TTQ_ENULL;
  return segmented_workspace(prm, n_segments, seg_offsets, bytes);
}

int ttq_linear_segmented(const ttq_params* prm, int64_t n_segments,
                         const int64_t* seg_offsets, const void* W,
                         const void* X, const void* B, const void* A, float* Y,
                         uint8_t* codes_out, float* scales_out, float* mins_out,
                         float* dhalf_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return segmented_impl(prm, n_segments, seg_offsets, W, X, B, A, Y, codes_out,
                        scales_out, mins_out, dhalf_out, workspace,
                        workspace_bytes, stream);
}

int ttq_path(const ttq_params* prm, int64_t n_requests) {
  const int st = validate_params(prm, n_requests);
  if (st != TTQ_OK) return st;
  return make_plan(prm, n_requests < 1 ? 1 : n_requests).path;
}

int ttq_packed_row_bytes(const ttq_params* prm, int64_t* bytes) {
  if (!bytes || !prm) return TTQ_ENULL;
  const ttq_params q = quantize_view(prm);
  return validate_packed(prm, q, bytes);
}

int ttq_quantize_workspace_bytes(const ttq_params* prm, size_t* bytes) {
  if (!bytes || !prm) return TTQ_ENULL;
  const ttq_params q = quantize_view(prm);
  int64_t rb = 0;
  const int st = validate_packed(prm, q, &rb);
  if (st != TTQ_OK) return st;
  *bytes = make_quantize_plan(q).total;
  return TTQ_OK;
}

int ttq_qmatmul_workspace_bytes(const ttq_params* prm, size_t* bytes) {
  if (!bytes || !prm) return TTQ_ENULL;
  const ttq_params q = qmatmul_view(prm);
  int64_t rb = 0;
  const int st = validate_packed(prm, q, &rb);
  if (st != TTQ_OK) return st;
  *bytes = make_qmatmul_plan(q, container_bits(q.bits)).total;
  return TTQ_OK;
}

int ttq_quantize(const ttq_params* prm, const void* W, const void* X,
                 uint8_t* codes, float* scales, float* mins, float* dhalf_inv,
                 float* dhalf_out, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return quantize_impl(prm, W, X, codes, scales, mins, dhalf_inv, dhalf_out,
                       workspace, workspace_bytes, stream);
}

int ttq_qmatmul(const ttq_params* prm, const uint8_t* codes,
                const float* scales, const float* mins, const float* dhalf_inv,
                const void* X, const void* B, const void* A, float* Y,
                void* workspace, size_t workspace_bytes, void* stream) {
  return qmatmul_impl(prm, codes, scales, mins, dhalf_inv, X, B, A, Y,
                      workspace, workspace_bytes, stream);
}

int ttq_lowrank_pca_workspace_bytes(const ttq_params* prm, int32_t iters,
                                    size_t* bytes) {
  if (!bytes) return TTQ_ENULL;
  const int st = validate_pca(prm, iters);
  if (st != TTQ_OK) return st;
  *bytes = make_pca_plan(prm).total;
  return TTQ_OK;
}

int ttq_lowrank_pca(const ttq_params* prm, int32_t iters, const void* W,
                    const void* X, const float* Omega, void* B_out,
                    void* A_out, void* Wres_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return pca_impl(prm, iters, W, X, Omega, B_out, A_out, Wres_out, workspace,
                  workspace_bytes, stream);
}

const char* ttq_status_string(int status) {
  switch (status) {
    case TTQ_OK: return "ok";
    case TTQ_EINVAL: return "invalid argument (size or scalar out of range)";
    case TTQ_ENULL: return "required pointer is NULL";
    case TTQ_EALIGN: return "pointer not aligned as required";
    case TTQ_EWORKSPACE: return "workspace too small";
    case TTQ_EUNSUPPORTED: return "valid but unsupported configuration";
    case TTQ_EHIP: return "HIP runtime error (see ttq_last_hip_error)";
    default: return "unknown status";
  }
}

int ttq_last_hip_error(void) { return g_last_hip_error; }

const char* ttq_version(void) { return "ttq-gfx950 0.1.0"; }

int ttq_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || bytes > (int64_t(1) << 40)) return TTQ_EINVAL;
  if (bytes == 0) return TTQ_OK;
  if (!src || !sink) return TTQ_ENULL;
  if (misaligned(src, 16) || misaligned(sink, 4)) return TTQ_EALIGN;
  if (inject_hip_error()) return TTQ_EHIP;
  return run(K_STREAM_READ, static_cast<hipStream_t>(stream),
             [&](const Launch& L) { return launch_stream_read(src, bytes, sink, L); });
}

int ttq_timing_enable(int on) {
  g_timing.enabled = on != 0;
  return TTQ_OK;
}

int ttq_timing_reset(void) {
  for (int k = 0; k < K_NUM_KINDS; ++k) {
    for (auto& pr : g_timing.pending[k]) {
      (void)hipEventSynchronize(pr.second);
      g_timing.pool.push_back(pr.first);
      g_timing.pool.push_back(pr.second);
    }
    g_timing.pending[k].clear();
    g_timing.total_ms[k] = 0.0;
    g_timing.launches[k] = 0;
  }
  return TTQ_OK;
}

int ttq_kernel_count(void) { return K_NUM_KINDS; }

const char* ttq_kernel_name(int kernel) {
  if (kernel < 0 || kernel >= K_NUM_KINDS) return nullptr;
  return kKernelNames[kernel];
}

int ttq_timing_query(int kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= K_NUM_KINDS) return TTQ_EINVAL;
  if (!total_ms || !launches) return TTQ_ENULL;
  for (auto& pr : g_timing.pending[kernel]) {
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return TTQ_EHIP;
    }
    g_timing.total_ms[kernel] += ms;
    g_timing.launches[kernel] += 1;
    g_timing.pool.push_back(pr.first);
    g_timing.pool.push_back(pr.second);
  }
  g_timing.pending[kernel].clear();
  *total_ms = g_timing.total_ms[kernel];
  *launches = g_timing.launches[kernel];
  return TTQ_OK;
}

}  // extern "C"
