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
// Layout: one workgroup per (sequence, head, d-slice). With many splits the
// head dimension is cut into ND = 4 slices so that more workgroups share the
// partial traffic. Inside a workgroup, thread (s, f) of 32 split lanes x FL
// d-lanes sums splits s, s + 32, ... for 4 consecutive d values (one slice of
// 32) or 16 (one slice of 128: 256 threads instead of 1024, so a CU holds
// four times as many rows at once), with the loads of U splits in flight at
// a time (with several slices, the first U before the maximum is known); the
// 32 lane sums are then added by a fixed tree: lane exchanges inside each
// wave, then the 4 waves in order through LDS.
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

// x of the lane R places round inside each 16-lane row (a DPP row
// rotation); for R = 8 that is lane l ^ 8.
template <int R>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + R, 0xf, 0xf, false));
}
// Maximum over the 64 lanes of a wave, by vector-ALU lane exchanges.
__device__ __forceinline__ float wave_max(float x) {
  float lo, hi;
  swap_halves(x, lo, hi);
  x = fmaxf(lo, hi);
  swap_rows16(x, lo, hi);
  x = fmaxf(lo, hi);
  // rotations of each 16-lane row by 8, 4, 2, 1
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  return fmaxf(x, row_ror<1>(x));
}
// Sum of x over lanes l, l ^ 8, l ^ 16, l ^ 32 of a wave (lane bits 3-5),
// as a fixed tree; every lane gets the same bits (each step adds two values,
// and floating-point addition of two values is commutative).
__device__ __forceinline__ float sum_lanes_8_16_32(float x) {
  x += row_ror<8>(x);
  float lo, hi;
  swap_rows16(x, lo, hi);
  x = lo + hi;
  swap_halves(x, lo, hi);
  return lo + hi;
}

// ND: d-slices per (sequence, head); each slice is kD / ND values, handled
// by FL = kD / ND / (4 V) d-lanes of V float4 each and kSL = 32 split lanes
// (FL * 32 threads: 256 in both layouts used). Split lane s sums splits s,
// s + 32, s + 64, ... in that order, with U partials in flight, and the 32
// lane sums are added by the same fixed tree in both layouts. The
// summation order of a row therefore depends only on its own split count,
// never on ND, on the batch or on max_splits: with a split length that does
// not depend on the batch, every row's bits are batch-invariant ("Decode
// attention: FlashDecoding, split-K, paged kernels", section "Split-K breaks
// bitwise reproducibility": fix the split tile so the count is a function of
// the sequence length alone).
constexpr int kSL = 32;

template <int DT, int ND, int U, int V>
__global__ __launch_bounds__(kD / ND / (4 * V) * kSL) void merge_kernel(MergeParams p) {
  using E = Elem<DT>;
  constexpr int kSlice = kD / ND;
  constexpr int FL = kSlice / (4 * V);
  constexpr int NT = FL * kSL;
  constexpr int NW = NT / 64;
  static_assert(FL == 8 && NW == 4, "the lane tree below takes 8 d-lanes and 4 waves of split lanes");
  __shared__ float red_m[NW];
  // per wave and d-lane: its 8 split lanes' sums of O~ (4V values) and l
  __shared__ __attribute__((aligned(16))) float red_w[NW][FL][4 * V + 4];

  const int bh = blockIdx.x;
  const int d0 = blockIdx.y * kSlice;
  const int b = bh / p.h;
  const int tid = threadIdx.x;
#ifdef ATTN_DEVICE_CHECKS
  const size_t part_rows = (size_t)p.B * p.h * p.max_splits;
#endif
  const int s_len = ATTN_IN_RANGE(p.seq_lens + b, 4, p.seq_lens, (size_t)p.B * 4, kSiteMrgLens) ? p.seq_lens[b] : 0;
  const int n = s_len <= 0 ? 0 : min(p.max_splits, (s_len + p.chunk - 1) / p.chunk);
  const size_t base = (size_t)bh * p.max_splits;

  // With several d-slices (many splits, few rows: latency decides) the
  // first U splits of each lane are loaded before the split count and the
  // maximum are known, so they are in registers when the maximum arrives:
  // rows up to max_splits lie inside the partial buffers, and those past the
  // valid count are masked once it is known (their contents are never used).
  // The merge then waits for one round trip instead of three. With one slice
  // (many rows: bytes decide) only valid rows are read, after the maximum.
  constexpr int U0 = ND > 1 ? U : 0;
  const int lim = ND > 1 ? p.max_splits : n;
  const int sl = tid / FL;
  const int d = (tid % FL) * 4 * V;
  float li0[U0 > 0 ? U0 : 1], mi0[U0 > 0 ? U0 : 1];
  f32x4 oi0[U0 > 0 ? U0 : 1][V];
#pragma unroll
  for (int u = 0; u < U0; ++u) {
    const int i = sl + u * kSL;
    const bool in = i < lim && ATTN_IN_RANGE(p.part_l + base + i, 4, p.part_l, part_rows * 4, kSiteMrgPartML) &&
                    ATTN_IN_RANGE(p.part_m + base + i, 4, p.part_m, part_rows * 4, kSiteMrgPartML);
    li0[u] = in ? p.part_l[base + i] : 0.f;
    mi0[u] = in ? p.part_m[base + i] : -INFINITY;
#pragma unroll
    for (int c = 0; c < V; ++c)
      oi0[u][c] = in && ATTN_IN_RANGE(&p.part_o[(base + i) * kD + d0 + d + 4 * c], 16, p.part_o, part_rows * kD * 4,
                                      kSiteMrgPartO)
                      ? *reinterpret_cast<const f32x4*>(&p.part_o[(base + i) * kD + d0 + d + 4 * c])
                      : f32x4{};
  }
  float mloc = -INFINITY;
  if (U0 * kSL >= lim) {
    // the preloaded rows are every split row: the maximum comes from them
#pragma unroll
    for (int u = 0; u < U0; ++u)
      if (sl + u * kSL < n && li0[u] > 0.f) mloc = fmaxf(mloc, mi0[u]);
  } else {
    for (int i = tid; i < lim; i += NT) {
      if (!(ATTN_IN_RANGE(p.part_m + base + i, 4, p.part_m, part_rows * 4, kSiteMrgPartML) &&
            ATTN_IN_RANGE(p.part_l + base + i, 4, p.part_l, part_rows * 4, kSiteMrgPartML)))
        continue;
      const float mi = p.part_m[base + i];
      if (i < n && p.part_l[base + i] > 0.f) mloc = fmaxf(mloc, mi);
    }
  }
  mloc = wave_max(mloc);
  if ((tid & 63) == 0) red_m[tid >> 6] = mloc;
  __syncthreads();
  float big = red_m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) big = fmaxf(big, red_m[w]);

  uint16_t* op = p.o + (size_t)bh * kD + d0;
  if (big == -INFINITY) {   // no visible key in any split: zero output
    if (tid < kSlice / 2 && ATTN_IN_RANGE(op + 2 * tid, 4, p.o, (size_t)p.B * p.h * kD * 2, kSiteMrgO))
      reinterpret_cast<uint32_t*>(op)[tid] = 0u;
    if (tid == 0 && blockIdx.y == 0 && p.lse != nullptr &&
        ATTN_IN_RANGE(p.lse + bh, 4, p.lse, (size_t)p.B * p.h * 4, kSiteMrgLse))
      p.lse[bh] = -INFINITY;
    return;
  }

  f32x4 acc[V];
#pragma unroll
  for (int c = 0; c < V; ++c) acc[c] = f32x4{};
  float lacc = 0.f;
#pragma unroll
  for (int u = 0; u < U0; ++u) {
    if (sl + u * kSL < n && li0[u] > 0.f) {
      const float w = fast_exp2((mi0[u] - big) * kLog2e);
      lacc += w * li0[u];
#pragma unroll
      for (int c = 0; c < V; ++c) acc[c] += w * oi0[u][c];
    }
  }
  for (int i0 = sl + U0 * kSL; i0 < n; i0 += U * kSL) {
    float li[U], mi[U];
    f32x4 oi[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kSL;
      const bool ok = i < n && ATTN_IN_RANGE(p.part_l + base + i, 4, p.part_l, part_rows * 4, kSiteMrgPartML) &&
                      ATTN_IN_RANGE(p.part_m + base + i, 4, p.part_m, part_rows * 4, kSiteMrgPartML);
      li[u] = ok ? p.part_l[base + i] : 0.f;
      mi[u] = ok ? p.part_m[base + i] : -INFINITY;
#pragma unroll
      for (int c = 0; c < V; ++c)
        oi[u][c] = ok && ATTN_IN_RANGE(&p.part_o[(base + i) * kD + d0 + d + 4 * c], 16, p.part_o,
                                       part_rows * kD * 4, kSiteMrgPartO)
                       ? *reinterpret_cast<const f32x4*>(&p.part_o[(base + i) * kD + d0 + d + 4 * c])
                       : f32x4{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (li[u] > 0.f) {
        const float w = fast_exp2((mi[u] - big) * kLog2e);
        lacc += w * li[u];
#pragma unroll
        for (int c = 0; c < V; ++c) acc[c] += w * oi[u][c];
      }
    }
  }
  // The 32 split lanes' sums: the 8 of each wave by lane exchanges (split
  // lane bits are lane bits 3-5), then the 4 waves in order through LDS.
#pragma unroll
  for (int c = 0; c < V; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[c][e] = sum_lanes_8_16_32(acc[c][e]);
  lacc = sum_lanes_8_16_32(lacc);
  const int wave = tid >> 6, wl = tid & 63;
  if (wl < FL) {
#pragma unroll
    for (int c = 0; c < V; ++c) *reinterpret_cast<f32x4*>(&red_w[wave][wl][4 * c]) = acc[c];
    red_w[wave][wl][4 * V] = lacc;
  }
  __syncthreads();
  if (tid < FL) {
    f32x4 o[V];
    float l_all = red_w[0][tid][4 * V];
#pragma unroll
    for (int c = 0; c < V; ++c) o[c] = *reinterpret_cast<const f32x4*>(&red_w[0][tid][4 * c]);
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      l_all += red_w[w][tid][4 * V];
#pragma unroll
      for (int c = 0; c < V; ++c) o[c] += *reinterpret_cast<const f32x4*>(&red_w[w][tid][4 * c]);
    }
    const float inv = 1.f / l_all;
#pragma unroll
    for (int c = 0; c < V; ++c) {
      const f32x4 q = o[c] * inv;
      if (ATTN_IN_RANGE(op + tid * 4 * V + 4 * c, 8, p.o, (size_t)p.B * p.h * kD * 2, kSiteMrgO))
        store8(op + tid * 4 * V + 4 * c, u32x2{E::pack2(q[0], q[1]), E::pack2(q[2], q[3])});
    }
    if (tid == 0 && blockIdx.y == 0 && p.lse != nullptr &&
        ATTN_IN_RANGE(p.lse + bh, 4, p.lse, (size_t)p.B * p.h * 4, kSiteMrgLse))
      p.lse[bh] = big + fast_log2(l_all) * kLn2;
  }
}

template <int DT>
hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  // Many splits and few (sequence, head) pairs: cut d into 4 slices so that
  // more workgroups share the partial traffic (same bits as one slice).
  if (p.max_splits >= 64 && (long)p.B * p.h < 1024) {
    hipLaunchKernelGGL((merge_kernel<DT, 4, 8, 1>), dim3((unsigned)(p.B * p.h), 4), dim3(kD / 4 / 4 * kSL), 0, stream, p);
  } else {
    // One split in flight per lane: 46 VGPRs instead of 100 with four, so
    // 9 workgroups per CU are resident (the LDS's limit) instead of 5 (the
    // register file's), and with many rows the
    // occupancy matters more than the loads in flight (same bits: the
    // summation order does not depend on U). Interleaved, HIP-graph timed:
    // 7.0 -> 5.8 us on the 64-sequence paged decode's partials (13 splits),
    // 11.8 -> 9.1 us with 128 heads and 8 splits, 13.8 -> 13.0 us with 150
    // splits.
    hipLaunchKernelGGL((merge_kernel<DT, 1, 1, 4>), dim3((unsigned)(p.B * p.h), 1), dim3(kD / 16 * kSL), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

ATTN_DEFINE_CHECK_READER(merge)

hipError_t merge_states(const float* part_o, const float* part_m, const float* part_l,
                        const int32_t* seq_lens, int chunk_keys, int B, int h, int max_splits,
                        void* o, float* lse, int dtype, hipStream_t stream) {
  MergeParams p{part_o, part_m, part_l, seq_lens, static_cast<uint16_t*>(o), lse, B, h, max_splits, chunk_keys};
  if (B == 0 || h == 0) return hipSuccess;
  if (dtype == ATTN_DTYPE_BF16) return launch_merge<ATTN_DTYPE_BF16>(p, stream);
  return launch_merge<ATTN_DTYPE_F16>(p, stream);
}

}  // namespace attn
