// Row copies for continuous batching: requests of different lengths packed
// one after another in X [sum T_r][d] are computed as batches of requests of
// one padded length.  The pages leave open how scales are derived when one
// batch mixes requests ("Test-time quantization: quantising on the fly with
// no calibration dataset", lo0 blog, section "What we have not covered");
// here every request keeps its own statistics, as for the batched call.
//
//   gather:  dst[r][t][:] = t < len[r] ? src[off[r] + t][:] : 0,  t < Tpad
//   scatter: dst[off[r] + t][:] = src[r][t][:],                  t < len[r]
//
// Zero tokens leave the L_p norms unchanged (they add exact zeros to the
// channel sums) and their output rows are dropped, so a padded request gives
// the same D, codes and Y rows as the request alone.  One workgroup copies
// one row with 16-byte accesses (4-byte ones when the row is not a multiple
// of 16 bytes).
#include "ttq_internal.h"

namespace ttq {

namespace {

template <int VB>
__global__ __launch_bounds__(256) void k_seg_copy(SegCopyArgs a) {
  const int r = blockIdx.y;
  const int64_t t = blockIdx.x;
  const int64_t len = a.len[r];
  if (a.scatter && t >= len) return;
  const int64_t row_bytes = a.row_bytes;
  const unsigned char* src;
  unsigned char* dst;
  if (a.scatter) {
    src = static_cast<const unsigned char*>(a.src) + ((int64_t)r * a.Tpad + t) * row_bytes;
    dst = static_cast<unsigned char*>(a.dst) + (a.off[r] + t) * row_bytes;
  } else {
    src = t < len ? static_cast<const unsigned char*>(a.src) + (a.off[r] + t) * row_bytes
                  : nullptr;
    dst = static_cast<unsigned char*>(a.dst) + ((int64_t)r * a.Tpad + t) * row_bytes;
  }
  for (int64_t i = (int64_t)threadIdx.x * VB; i < row_bytes; i += 256 * VB) {
    if (VB == 16) {
      const u32x4 v = src ? *(const u32x4*)(src + i) : u32x4{0u, 0u, 0u, 0u};
      *(u32x4*)(dst + i) = v;
    } else {
      const unsigned v = src ? *(const unsigned*)(src + i) : 0u;
      *(unsigned*)(dst + i) = v;
    }
  }
}

}  // namespace

hipError_t launch_seg_copy(const SegCopyArgs& a, const Launch& L) {
  if (a.n <= 0 || a.Tpad <= 0 || a.row_bytes <= 0) return hipSuccess;
  if (a.n > kSegMax || a.row_bytes % 4 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.Tpad, (unsigned)a.n), blk(256);
  if (a.row_bytes % 16 == 0) return ext_launch(k_seg_copy<16>, grid, blk, 0, L, a);
  return ext_launch(k_seg_copy<4>, grid, blk, 0, L, a);
}

}  // namespace ttq
