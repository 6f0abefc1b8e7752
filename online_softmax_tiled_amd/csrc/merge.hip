// Decode stage 2 for gfx950: merge the split-KV partial states of each
// (sequence, query head) into the normalised output and its LSE.
//
// "Decode attention: FlashDecoding, split-K, paged kernels", the stage-2
// reduction described in section "Where GQA enters": take the largest
// reference maximum M over the valid splits, rescale each split's l_i and
// O~_i by exp(m_i - M), sum, divide once, and give zero when the total mass
// is zero; no K or V is read again. The valid split count of sequence b is
// recomputed from its length exactly as the producer computes it (section
// "CUDA graphs need the split count pinned": producer and reducer must
// agree on which partial rows exist). An empty split (m_i = -inf or l_i = 0)
// contributes nothing and never forms -inf - (-inf) ("Merge normalized
// attention without averaging tile outputs", paragraph on fully masked
// tiles).
//
// One workgroup of 256 threads per (sequence, head): 8 groups of 32 threads
// take every 8th split, each thread 4 consecutive d values; the 8 group sums
// are combined through LDS.
#include "common.h"

namespace attn {
namespace {

constexpr int kD = 128;

struct MergeParams {
  const float* part_o;
  const float* part_m;
  const float* part_l;
  const int32_t* seq_lens;
  uint16_t* o;
  float* lse;
  int B, h, max_splits, chunk;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

template <int DT>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  using E = Elem<DT>;
  __shared__ float red_m[4];
  __shared__ __attribute__((aligned(16))) float red_o[8][kD];
  __shared__ float red_l[8];

  const int bh = blockIdx.x;
  const int b = bh / p.h;
  const int tid = threadIdx.x;
  const int s_len = p.seq_lens[b];
  const int n = s_len <= 0 ? 0 : min(p.max_splits, (s_len + p.chunk - 1) / p.chunk);
  const size_t base = (size_t)bh * p.max_splits;

  float mloc = -INFINITY;
  for (int i = tid; i < n; i += 256) {
    const float mi = p.part_m[base + i];
    if (p.part_l[base + i] > 0.f) mloc = fmaxf(mloc, mi);
  }
  mloc = wave_max(mloc);
  if ((tid & 63) == 0) red_m[tid >> 6] = mloc;
  __syncthreads();
  const float big = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  uint16_t* op = p.o + (size_t)bh * kD;
  if (big == -INFINITY) {   // no visible key in any split: zero output
    if (tid < kD / 2) reinterpret_cast<uint32_t*>(op)[tid] = 0u;
    if (tid == 0 && p.lse != nullptr) p.lse[bh] = -INFINITY;
    return;
  }

  const int grp = tid >> 5;
  const int d = (tid & 31) * 4;
  f32x4 acc = f32x4{};
  float lacc = 0.f;
  for (int i = grp; i < n; i += 8) {
    const float li = p.part_l[base + i];
    if (!(li > 0.f)) continue;
    const float w = fast_exp2((p.part_m[base + i] - big) * kLog2e);
    lacc += w * li;
    acc += w * *reinterpret_cast<const f32x4*>(&p.part_o[(base + i) * kD + d]);
  }
  *reinterpret_cast<f32x4*>(&red_o[grp][d]) = acc;
  if ((tid & 31) == 0) red_l[grp] = lacc;
  __syncthreads();
  if (tid < kD / 2) {
    float l_all = 0.f;
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) l_all += red_l[gi];
    const int dd = tid * 2;
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
      o0 += red_o[gi][dd];
      o1 += red_o[gi][dd + 1];
    }
    const float inv = 1.f / l_all;
    reinterpret_cast<uint32_t*>(op)[tid] = E::pack2(o0 * inv, o1 * inv);
    if (tid == 0 && p.lse != nullptr) p.lse[bh] = big + fast_log2(l_all) * kLn2;
  }
}

}  // namespace

hipError_t merge_states(const float* part_o, const float* part_m, const float* part_l,
                        const int32_t* seq_lens, int chunk_keys, int B, int h, int max_splits,
                        void* o, float* lse, int dtype, hipStream_t stream) {
  MergeParams p{part_o, part_m, part_l, seq_lens, static_cast<uint16_t*>(o), lse, B, h, max_splits, chunk_keys};
  if (B == 0 || h == 0) return hipSuccess;
  const dim3 grid((unsigned)(B * h));
  if (dtype == ATTN_DTYPE_BF16)
    hipLaunchKernelGGL(merge_kernel<ATTN_DTYPE_BF16>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<ATTN_DTYPE_F16>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
