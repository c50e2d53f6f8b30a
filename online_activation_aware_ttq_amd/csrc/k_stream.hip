// Plain streaming read of device memory: the measured ceiling of the
// one-token projection, which is one pass over W.  Same launch shape as that
// kernel (a workgroup of 16 waves per 16 weight rows of a 4096-channel row,
// i.e. per 128 KiB, each lane with 64 bytes in flight): every lane requests
// four 16-byte pieces, folds them into a 32-bit XOR as they arrive, and
// requests the next four; one XOR per workgroup leaves so that no load is
// elided.  Not part of the method.
#include "ttq_internal.h"

namespace ttq {

namespace {

constexpr int SR_THREADS = 1024;
constexpr int SR_INFLIGHT = 4;   // 16-byte loads per lane in flight

__global__ __launch_bounds__(SR_THREADS) void k_stream_read(const uint8_t* src,
                                                            int64_t bytes,
                                                            uint32_t* sink) {
  const int64_t b = blockIdx.x;
  const int64_t base = b * kStreamReadBlockBytes;
  const int64_t n = min((int64_t)kStreamReadBlockBytes, bytes - base);
  // the workgroup's bytes as one bounded buffer: pieces past the end read
  // zeros without traffic
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src + base, (uint32_t)n);
  const uint32_t tid = threadIdx.x;
  uint32_t x = 0u;
  constexpr uint32_t kStep = SR_THREADS * 16 * SR_INFLIGHT;
  for (uint32_t off = 0; off < (uint32_t)n; off += kStep) {
    u32x4 v[SR_INFLIGHT];
#pragma unroll
    for (int j = 0; j < SR_INFLIGHT; ++j)
      v[j] = buf_load16(r, off + (j * SR_THREADS + tid) * 16, 0);
#pragma unroll
    for (int j = 0; j < SR_INFLIGHT; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // fixed-order reduction: xor over the wave, then the waves in order
  __shared__ uint32_t red[SR_THREADS / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  if (tid == 0) {
    uint32_t y = 0u;
    for (int w = 0; w < SR_THREADS / 64; ++w) y ^= red[w];
    sink[b] = y;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                              const Launch& L) {
  const int64_t nblk = (bytes + kStreamReadBlockBytes - 1) / kStreamReadBlockBytes;
  if (nblk == 0) return hipSuccess;
  return ext_launch(k_stream_read, dim3((unsigned)nblk), dim3(SR_THREADS), 0, L,
                    (const uint8_t*)src, bytes, sink);
}

}  // namespace ttq
