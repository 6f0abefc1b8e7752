// Read-rate calibration for the HBM-bound kernels: reads a buffer once, as a
// plain stream, and writes one 32-bit value per workgroup so the loads cannot
// be dropped. Each workgroup reads one contiguous chunk with 16-byte
// non-temporal loads, four in flight per thread -- the access pattern of the
// decode kernels' K/V reads. Timing it on the decode step's own byte count
// gives the read rate attainable at that size (launch, first-byte latency
// and drain included), which is the floor the split-KV decode is compared
// with.
#include "common.h"

namespace attn {
namespace {

constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* src, uint64_t n16,
                                                                     uint64_t per_wg, uint32_t* out) {
  const uint64_t lo = (uint64_t)blockIdx.x * per_wg;
  const uint64_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
  uint32_t acc = 0;
  for (uint64_t i = lo + threadIdx.x; i < hi; i += 4 * kStreamThreads) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t k = i + (uint64_t)u * kStreamThreads;
      v[u] = k < hi && ATTN_IN_RANGE(src + k, 16, src, n16 * 16, kSiteStream) ? load16_nt(src + k)
                                                                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // one value per workgroup: xor over the threads
  __shared__ uint32_t red[kStreamThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

#ifdef ATTN_DEVICE_CHECKS
// The checker's own test: one address inside a 64-byte extent and one past
// it, tested and not accessed.
__global__ void check_selftest_kernel(const uint8_t* base) {
  if (threadIdx.x != 0) return;
  (void)ATTN_IN_RANGE(base + 56, 8, base, 64, kSiteSelfTestIn);
  (void)ATTN_IN_RANGE(base + 60, 8, base, 64, kSiteSelfTestOut);
}
#endif

}  // namespace

ATTN_DEFINE_CHECK_READER(stream)

#ifdef ATTN_DEVICE_CHECKS
hipError_t check_selftest(const void* base, hipStream_t stream) {
  hipLaunchKernelGGL(check_selftest_kernel, dim3(1), dim3(64), 0, stream, static_cast<const uint8_t*>(base));
  return hipGetLastError();
}
#endif

// chunks: workgroups (each reads bytes / chunks, rounded up to 16 bytes).
hipError_t stream_read(const void* src, uint64_t bytes, int chunks, uint32_t* out, hipStream_t stream) {
  const uint64_t n16 = bytes / 16;
  const uint64_t per = (n16 + chunks - 1) / chunks;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)chunks), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4*>(src), n16, per, out);
  return hipGetLastError();
}

}  // namespace attn
