/*
 * ttq.h -- C ABI of the TTQ linear projection on AMD Instinct MI355X (gfx950).
 *
 * TTQ (activation-aware test-time quantization, arXiv:2603.19296) quantizes
 * the weights of a linear layer on the fly from the activations of the
 * current call, with no calibration data and no state kept between calls.
 * For activations X (d input channels x T tokens) and weights W (d' x d)
 * one call computes
 *
 *   n_i      = ||X_{i,:}||_p                        L_p norm of channel i
 *   D_ii     = (n_i + lambda)^alpha                 damped diagonal
 *   W_hat    = Q[W D^{1/2}] D^{-1/2}                group quantize-dequantize
 *   Y        = W_hat X + B (A X)                    plus the static low rank
 *
 * as defined in "TTQ: Activation-Aware Test-Time Quantization to Accelerate
 * LLM Inference On The Fly" (gist.science zh summary, Sec. 2.1 for D and
 * W_hat, Sec. 2.2 for the low-rank term; the nl and it summaries, Sec. 2,
 * restate both).  Q is the asymmetric b-bit affine quantizer of the blog
 * "Test-time quantization: quantising on the fly with no calibration
 * dataset", section "The maths that matter", applied to groups of `group`
 * consecutive input channels of each output row, with a min-anchored real
 * zero point: s = (max - min)/(2^b - 1), q = clamp(rint((u - min)/s)),
 * u_hat = min + s q.  Codes are decided in IEEE float32:
 *   dh = float32(D^{1/2}); u = w*dh; s = (max-min)/N; inv = 1/s (0 if s=0);
 *   t = (u - min)*inv; q = clamp(rint_half_even(t), 0, N)
 * with every operation correctly rounded and no fused multiply-add.  The
 * statistics (norms and powers) are evaluated in float64.
 *
 * Memory layout (all row-major, bfloat16 = raw 16-bit patterns):
 *   W  [d_out][d]      bf16    (nn.Linear weight layout)
 *   X  [T][d]          bf16    (token-major; batched: [R][T][d])
 *   B  [d_out][rank]   bf16    A [rank][d] bf16   (both NULL if rank == 0)
 *   Y  [T][d_out]      float32 (batched: [R][T][d_out])
 *
 * Ownership and ordering: every pointer is caller-owned device memory (or
 * NULL where optional).  The library never allocates, frees or synchronizes
 * on the calling path: it validates arguments on the host, enqueues kernels
 * on `stream` (a hipStream_t; NULL is the null stream) and returns.  Device
 * faults surface at the caller's next synchronization.  Results are
 * deterministic: identical inputs give bit-identical outputs.
 *
 * Accuracy of Y: the contraction accumulates in float32.  Its activation
 * operand x' = x D^{-1/2} is float32 for one token, fp16 scaled by a power
 * of two per (group, token) for 2..16 tokens (any float32 magnitude), and
 * bf16 above; above 128 tokens the dequantized weights are rounded once to
 * bf16 and contracted with the bf16 X.
 *
 * Errors: validation happens before anything is enqueued, so a negative
 * status means nothing was launched -- except TTQ_EHIP, which reports a
 * failed launch (some earlier kernels of the same call may have been
 * enqueued); the raw hipError_t is then available from ttq_last_hip_error().
 */
#ifndef TTQ_H_
#define TTQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  TTQ_OK = 0,
  TTQ_EINVAL = -1,       /* a size or scalar argument is out of range          */
  TTQ_ENULL = -2,        /* a required pointer is NULL                          */
  TTQ_EALIGN = -3,       /* a pointer is not aligned as required                */
  TTQ_EWORKSPACE = -4,   /* workspace smaller than ttq_workspace_bytes()        */
  TTQ_EUNSUPPORTED = -5, /* valid by the method, not supported by this library  */
  TTQ_EHIP = -100        /* a HIP runtime call failed; see ttq_last_hip_error() */
};

/* flags */
#define TTQ_FLAG_FORCE_FUSED 1u    /* use the single-pass fused path (T <= 128) */
#define TTQ_FLAG_FORCE_TWO_PHASE 2u /* quantize pass + GEMM, at any T            */

/* Quantizer formats (ttq_params.qformat).  The method derives the scale from
 * the activations and leaves the code format open (lo0 blog "Test-time
 * quantization: quantising on the fly with no calibration dataset", section
 * "What TTQ is NOT": orthogonal to INT4 or FP8; section "The maths that
 * matter" for the symmetric scale and the affine form with a zero point).
 * For one group of u = w D^{1/2} (float32, no fused operations, inv = 1/s or
 * 0 when s = 0, rint = round half to even):
 *   TTQ_QF_ASYM   s = (max - min)/N, q = clamp(rint((u - min) inv), 0, N),
 *                 u_hat = min + s q                 (N = 2^b - 1; default)
 *   TTQ_QF_SYM    s = max|u| / Z (Z = 2^{b-1} - 1, b >= 2),
 *                 k = clamp(rint(u inv), -Z, Z), u_hat = s k, code q = k + Z
 *   TTQ_QF_INTZP  lo = min(min u, 0), hi = max(max u, 0), s = (hi - lo)/N,
 *                 z = rint(lo inv), q = clamp(rint(u inv) - z, 0, N),
 *                 u_hat = s (q + z)   (integer zero point; zero is exact)
 *   TTQ_QF_FP8    b = 8: s = max|u| / 448, code = the OCP FP8 E4M3 pattern
 *                 of the nearest E4M3 value v (ties to even) of
 *                 clamp(u inv, -448, 448), u_hat = s v (the sign bit is
 *                 that of u inv, also when v is zero)
 * The per-group term stored beside the scales (mins_out, and the `mins` of
 * ttq_quantize / ttq_qmatmul) is the offset m with u_hat = m + s q for the
 * integer formats: the minimum (ASYM), -(Z s) (SYM), z s (INTZP), each
 * rounded once to float32; it is 0 for FP8, whose codes decode to E4M3
 * values.  Codes are decided exactly as stated; Y uses these stored terms. */
#define TTQ_QF_ASYM 0u
#define TTQ_QF_SYM 1u
#define TTQ_QF_INTZP 2u
#define TTQ_QF_FP8 3u

/* One projection's shape and the method's constants.
 *   d      input channels; >= 1 and a multiple of `group`
 *   d_out  output channels; >= 0
 *   T      tokens per request; >= 0 (T = 0: Y is empty, codes/scales are
 *          still produced from zero statistics)
 *   rank   low-rank r; 0 = no low-rank term; otherwise a multiple of 8, <= 1024
 *   bits   code width b in 1..8 (2..8 for TTQ_QF_SYM, 8 for TTQ_QF_FP8)
 *   group  group size along d: 32, 64, 128 or 256
 *   p      norm order, finite and > 0 (1 and 2 are exact; others use pow)
 *   lambda damping, finite and >= 0
 *   alpha  exponent, finite and >= 0 (0 gives D = I, i.e. plain RTN)
 *   flags  0, or one TTQ_FLAG_* path override
 *   qformat one of TTQ_QF_* (0 = the asymmetric quantizer)                   */
typedef struct ttq_params {
  int64_t d;
  int64_t d_out;
  int64_t T;
  int64_t rank;
  int32_t bits;
  int32_t group;
  double p;
  double lambda;
  double alpha;
  uint32_t flags;
  uint32_t qformat;
} ttq_params;

/* Device workspace, in bytes, that ttq_linear (n_requests = 1) or
 * ttq_linear_batched needs for these parameters.  Writes *bytes; returns a
 * status (the same validation as the compute calls, minus pointers). */
int ttq_workspace_bytes(const ttq_params* prm, int64_t n_requests,
                        size_t* bytes);

/* One TTQ linear call (one request).
 *   W, X             required (X may be NULL when T == 0); 16-byte aligned
 *   B, A             required iff rank > 0; 16-byte aligned
 *   Y                [T][d_out] float32; required iff T*d_out > 0; 4-byte aligned
 *   codes_out        optional [d_out][d] uint8 codes q
 *   scales_out       optional [d_out][d/group] float32 scales s
 *   mins_out         optional [d_out][d/group] float32 group offsets m (the
 *                    minima for TTQ_QF_ASYM; see TTQ_QF_*)
 *   dhalf_out        optional [d] float32 D^{1/2} as fed to the code decision
 *   workspace        device scratch of at least ttq_workspace_bytes(prm, 1);
 *                    256-byte aligned; contents need not be initialized and
 *                    are clobbered; must not be shared by concurrent calls
 *   stream           hipStream_t to enqueue on
 * Returns TTQ_OK or a negative status. */
int ttq_linear(const ttq_params* prm, const void* W, const void* X,
               const void* B, const void* A, float* Y, uint8_t* codes_out,
               float* scales_out, float* mins_out, float* dhalf_out,
               void* workspace, size_t workspace_bytes, void* stream);

/* R independent requests on one shared W (and B, A): each request has its
 * own statistics D computed from its own X (multitenant traffic).  X is
 * [R][T][d], Y [R][T][d_out]; the optional outputs gain a leading [R]
 * dimension.  n_requests = 0 is a valid no-op. */
int ttq_linear_batched(const ttq_params* prm, int64_t n_requests,
                       const void* W, const void* X, const void* B,
                       const void* A, float* Y, uint8_t* codes_out,
                       float* scales_out, float* mins_out, float* dhalf_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ---- allocation-free variant ----------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as ttq_linear_batched (n_requests = 1 is ttq_linear),
 * minus the workspace: the library takes it from a static device array of
 * TTQ_NOALLOC_SCRATCH_BYTES that every GPU it runs on holds until the process
 * ends (its address is looked up on the first call on each device, with that
 * device current).  The call allocates nothing, frees nothing and calls no
 * allocating routine.  All calls on one GPU share that GPU's array, which
 * keeps the last call's contents (no kernel needs it cleared): calls that
 * overlap on one GPU -- concurrent streams or threads -- race and must be
 * serialised by the caller.
 * Errors: as ttq_linear_batched, plus TTQ_EWORKSPACE when the call needs more
 * scratch than TTQ_NOALLOC_SCRATCH_BYTES (ttq_workspace_bytes gives the need;
 * checked on the host, nothing is enqueued), and TTQ_EHIP when the array's
 * address cannot be obtained. */
#define TTQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ttq_linear_noalloc(const ttq_params* prm, int64_t n_requests,
                       const void* W, const void* X, const void* B,
                       const void* A, float* Y, uint8_t* codes_out,
                       float* scales_out, float* mins_out, float* dhalf_out,
                       void* stream);

/* ---- continuous batching: requests of different lengths in one X --------
 * n_segments requests packed one after another: request i owns the token
 * rows seg_offsets[i] .. seg_offsets[i+1]-1 of X [T][d] and Y [T][d_out],
 * where prm->T is the total token count.  The pages leave open how scales
 * are derived when one batch mixes requests ("Test-time quantization:
 * quantising on the fly with no calibration dataset", lo0 blog, section "What
 * we have not covered"); here every request keeps its own statistics D, as
 * in ttq_linear_batched, and its codes, scales and Y rows equal those of
 * ttq_linear on that request alone, bit for bit (with a low-rank term, up to
 * 64 MiB of low-rank partial sums per batch).
 *   seg_offsets  host array of n_segments + 1 non-decreasing token offsets,
 *                seg_offsets[0] = 0, seg_offsets[n_segments] = prm->T;
 *                empty requests (equal offsets) are allowed
 *   optional outputs gain a leading [n_segments] dimension, as in
 *   ttq_linear_batched; all other arguments as for ttq_linear.
 * The requests of one length class (1; 2..16; 17..32; 33..64; 65..128
 * tokens; up to 64 at a time) are computed as one batch, shorter ones padded
 * with zero tokens (which leave the norms unchanged) through workspace copies
 * unless the batch is a run of consecutive requests of one length; when codes,
 * scales or D^{1/2} are asked for, a batch takes only consecutive requests.
 * Longer requests, or any request when a path flag is set, run alone.
 * n_segments = 0 is a no-op.
 * Errors: TTQ_ENULL for a NULL seg_offsets (n_segments > 0); TTQ_EINVAL for
 * offsets that do not start at 0, end at prm->T or decrease, and for the
 * conditions of ttq_linear_batched. */
int ttq_segmented_workspace_bytes(const ttq_params* prm, int64_t n_segments,
                                  const int64_t* seg_offsets, size_t* bytes);
int ttq_linear_segmented(const ttq_params* prm, int64_t n_segments,
                         const int64_t* seg_offsets, const void* W,
                         const void* X, const void* B, const void* A, float* Y,
                         uint8_t* codes_out, float* scales_out, float* mins_out,
                         float* dhalf_out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Which path a call with these parameters takes: 0 = fused single pass over
 * W (statistics kernel + one fused quantize/MFMA kernel), 1 = two phase
 * (statistics, quantize pass writing W_hat, MFMA GEMM), 2 = single launch
 * for one token (T = 1, d <= 12288, no path flag), 3 = two phase with the
 * weight tiles quantized inside the MFMA GEMM (129 <= T <= 256, d a
 * multiple of 128, group <= 128, no path flag; a call that asks for codes or
 * scales adds a pass over W that writes only them).  Paths 1 and 3 give
 * bit-identical Y.
 * Negative = status. */
int ttq_path(const ttq_params* prm, int64_t n_requests);

/* ---- quantize once per prompt, decode from the stored codes -------------
 * The statistics can be taken once per input prompt ("TTQ: Activation-Aware
 * Test-Time Quantization ...", nl summary, Sec. 2; zh summary, Sec. 3-4:
 * the speed-up comes from contracting stored low-bit weights, because
 * moving weights is the bottleneck).  ttq_quantize computes D from the
 * prompt's X and stores the codes, the per-group (s, min) and D^{-1/2};
 * ttq_qmatmul then computes, for the activations X of a later step,
 *   Y = X ((min + s q) D^{-1/2})^T + (X A^T) B^T
 * with those stored values (nothing is recomputed from the step's X).
 *
 * Code storage: each b-bit code takes the smallest container c of 1, 2, 4
 * or 8 bits that holds it; channel j of a row sits at bit (j*c) % 8 of byte
 * (j*c) / 8 of that row (least significant bits first).  A row takes
 * ttq_packed_row_bytes = d*c/8 bytes; d*c must be a multiple of 128 bits
 * (always true for the supported group sizes when c >= 4; checked). */

/* Bytes of one row of packed codes for these parameters (writes *bytes). */
int ttq_packed_row_bytes(const ttq_params* prm, int64_t* bytes);

/* Device workspace for ttq_quantize / ttq_qmatmul (writes *bytes). */
int ttq_quantize_workspace_bytes(const ttq_params* prm, size_t* bytes);
int ttq_qmatmul_workspace_bytes(const ttq_params* prm, size_t* bytes);

/* Quantize W for the prompt X ([T][d] bf16, T = prm->T >= 0; T = 0 gives
 * D from zero statistics, as in ttq_linear).
 *   codes       [d_out][row_bytes] packed codes, 16-byte aligned, required
 *   scales      [d_out][d/group] float32 s, required
 *   mins        [d_out][d/group] float32 group offsets m (minima for
 *               TTQ_QF_ASYM; see TTQ_QF_*), required
 *   dhalf_inv   [d] float32 D^{-1/2} = float32(1 / D^{1/2}), required
 *   dhalf_out   optional [d] float32 D^{1/2} as fed to the code decision
 * rank and the path flags are not read (the low-rank factors are used as
 * given by ttq_qmatmul); unknown flag bits are still TTQ_EINVAL.  Same
 * validation, alignment and error rules as ttq_linear otherwise. */
int ttq_quantize(const ttq_params* prm, const void* W, const void* X,
                 uint8_t* codes, float* scales, float* mins, float* dhalf_inv,
                 float* dhalf_out, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Y [T][d_out] float32 for the step activations X ([T][d] bf16, T =
 * prm->T) from the stored codes, scales, mins and dhalf_inv of ttq_quantize
 * (same d, d_out, bits, group and qformat: TTQ_QF_FP8 codes decode as E4M3
 * values, every other format as integers with the stored offsets, u_hat =
 * mins + scales * code).  B, A as in ttq_linear (rank = prm->rank).
 * codes 16-byte aligned, dhalf_inv 16-byte aligned, the rest as in
 * ttq_linear.  p, lambda, alpha and TTQ_FLAG_FORCE_FUSED are not used;
 * Routes: T = 1, a single kernel over the codes (unless x D^{-1/2} of the
 * token does not fit 128 KiB of LDS: d above about 30000); T <= 128, the
 * codes on the matrix cores; otherwise a GEMM that expands the codes to
 * bf16 weights tile by tile in LDS (d a multiple of 128), else a pass that
 * writes the expanded weights followed by a GEMM.  TTQ_FLAG_FORCE_TWO_PHASE
 * takes that last route at any T; both expansions give the same Y bits. */
int ttq_qmatmul(const ttq_params* prm, const uint8_t* codes,
                const float* scales, const float* mins, const float* dhalf_inv,
                const void* X, const void* B, const void* A, float* Y,
                void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text of a status code (static storage). */
const char* ttq_status_string(int status);

/* The hipError_t of the last failed HIP call on this thread (0 if none). */
int ttq_last_hip_error(void);

/* Library version string (static storage). */
const char* ttq_version(void);

/* ---- measurement ------------------------------------------------------
 * When enabled, every kernel the library launches is bracketed by a pair of
 * hipEvents recorded on the launch stream, and ttq_timing_query() sums
 * their elapsed times per kernel kind.  For measurement only: the timing
 * state is process-global and not thread-safe; query synchronizes on the
 * recorded events. */
int ttq_timing_enable(int on);
int ttq_timing_reset(void);
int ttq_kernel_count(void);
const char* ttq_kernel_name(int kernel);
int ttq_timing_query(int kernel, double* total_ms, int64_t* launches);

/* Plain streaming read, the measured ceiling of a one-pass kernel over W (not
 * part of the method): reads `bytes` bytes of device memory at `src` once,
 * in the launch shape of the one-token projection (one workgroup of 16
 * waves per 128 KiB, 64 bytes per lane in flight), and writes the 32-bit XOR
 * of each workgroup's words to sink[ceil(bytes / 131072)] (device memory)
 * so that no load is elided.  Timed as the kernel kind "stream_read".
 * `bytes` is a multiple of 16 (TTQ_EINVAL otherwise); `src` 16-byte and
 * `sink` 4-byte aligned (TTQ_EALIGN); both non-NULL when bytes > 0
 * (TTQ_ENULL).  Enqueued on `stream`. */
int ttq_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* ---- low-rank factors by PCA
 * The static low-rank factors of the projection are initialised by PCA, and
 * may be adapted online ("TTQ: Activation-Aware Test-Time Quantization ...",
 * nl summary, Sec. 2; it summary, Sec. 2; zh summary, Sec. 2.2); the pages
 * give no algorithm.  This call computes
 *   B  [d_out][rank] bf16: an orthonormal basis of the top-rank left
 *      principal subspace of M = W (T = 0), or of M = W D^{1/2} with D from
 *      the activations X (T > 0; p, lambda, alpha as in ttq_linear);
 *   A  [rank][d] bf16 = B^T W;
 *   Wres optional [d_out][d] bf16 = bf16(W - B A), computed from the bf16
 *      B and A, so that ttq_linear(Wres, X, B, A) projects with
 *      W ~ Q_D[Wres] + B A;
 * by randomized subspace iteration (Halko, Martinsson and Tropp, 2011):
 * Q = orth(M Omega), then `iters` times Z = orth(M^T Q), Q = orth(M Z), with
 * orth = CholeskyQR (float32 panels, float64 Cholesky; two passes for the
 * final basis, one for the intermediate panels), B = Q.  When M has rank
 * below `rank` (e.g. W = 0) the columns past the rank are not determined by
 * M: a column whose Gram pivot is at the float32 noise level (1e-5 of the
 * largest) is dropped, and in the first pass of the final basis replaced by
 * a pseudo-random column before the second pass,
 * so B is orthonormal in every case (A and Wres do not depend on the choice).
 *   prm     d, d_out >= 1; rank in {8, 16, 32, 64, 128}, <= min(d, d_out);
 *           T >= 0 (T > 0 needs d % 8 == 0); bits, group, flags and qformat
 *           are not read
 *   iters   power iterations, 0..16
 *   W       [d_out][d] bf16; X [T][d] bf16 (T > 0; NULL otherwise)
 *   Omega   [d][rank] float32, the caller's Gaussian test matrix
 *   workspace at least ttq_lowrank_pca_workspace_bytes, 256-byte aligned
 * All pointers 16-byte aligned device memory.  Same error rules as
 * ttq_linear; the result is deterministic for given inputs. */
int ttq_lowrank_pca_workspace_bytes(const ttq_params* prm, int32_t iters,
                                    size_t* bytes);
int ttq_lowrank_pca(const ttq_params* prm, int32_t iters, const void* W,
                    const void* X, const float* Omega, void* B_out,
                    void* A_out, void* Wres_out, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTQ_H_ */
