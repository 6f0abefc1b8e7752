// Two-operand merge in (O, LSE) form for gfx950: combine the normalised
// attention outputs of two disjoint key ranges of the same query rows (a
// cascade's shared prefix and per-request suffix, or two context-parallel
// shards) into the output over their union.
//
// "Naive attention and the online softmax", sections "The state that gets
// passed around is the log-sum-exp" and "Scale first, then multiply": with
// M = max(LSE_a, LSE_b) the weights w = exp(LSE - M) are divided by their
// sum before they multiply O, so the result is a convex combination and no
// huge intermediate is formed; LSE = M + ln(w_a + w_b). Section "The base case
// is a NaN factory": an LSE of +inf (the empty-row convention of some
// producers) is read as -inf, a side with LSE = -inf contributes nothing and
// its O is never read, and when both sides are empty the output is zeros
// with LSE = -inf ("Merge normalized attention without averaging tile
// outputs", last paragraph).
//
// Layout: rows of d_h = 128 elements; 16 lanes per row, 16 bytes each, 16
// rows per 256-thread workgroup. Every element is read and written by the
// same lane, so the output may alias either input. Loads and stores carry
// the non-temporal hint (each byte is touched once): 6.0 TB/s against 5.7
// without it on the [1, 32, 8192, 128] shape.
#include "common.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kRowsPerWg = 16;

struct MergeLseParams {
  const uint16_t* o_a;
  const float* lse_a;
  const uint16_t* o_b;
  const float* lse_b;
  uint16_t* o;
  float* lse;
  int rows;
};

template <int DT>
__global__ __launch_bounds__(256) void merge_lse_kernel(MergeLseParams p) {
  using E = Elem<DT>;
  const int row = blockIdx.x * kRowsPerWg + (threadIdx.x >> 4);
  if (row >= p.rows) return;
  const int c = threadIdx.x & 15;
  const bool rows_ok = ATTN_IN_RANGE(p.lse_a + row, 4, p.lse_a, (size_t)p.rows * 4, kSiteMlseLse) &&
                       ATTN_IN_RANGE(p.lse_b + row, 4, p.lse_b, (size_t)p.rows * 4, kSiteMlseLse);
  if (!rows_ok) return;
  float la = p.lse_a[row];
  float lb = p.lse_b[row];
  la = la == INFINITY ? -INFINITY : la;
  lb = lb == INFINITY ? -INFINITY : lb;
  const float big = fmaxf(la, lb);
  const size_t off = (size_t)row * kD + c * 8;
  u32x4 out = u32x4{0u, 0u, 0u, 0u};
  float lse_out = -INFINITY;
  if (big != -INFINITY) {
    // exp(l - M) = 2^((l - M) log2 e); an empty side gets weight exactly 0.
    const float ea = la == -INFINITY ? 0.f : fast_exp2((la - big) * kLog2e);
    const float eb = lb == -INFINITY ? 0.f : fast_exp2((lb - big) * kLog2e);
    const float tot = ea + eb;
    const float pa = ea / tot;
    const float pb = eb / tot;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if (ea > 0.f && ATTN_IN_RANGE(p.o_a + off, 16, p.o_a, (size_t)p.rows * kD * 2, kSiteMlseIn)) {
      const u32x4 va = load16_nt(p.o_a + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += pa * E::to_f32((uint16_t)(va[i] & 0xffffu));
        acc[2 * i + 1] += pa * E::to_f32((uint16_t)(va[i] >> 16));
      }
    }
    if (eb > 0.f && ATTN_IN_RANGE(p.o_b + off, 16, p.o_b, (size_t)p.rows * kD * 2, kSiteMlseIn)) {
      const u32x4 vb = load16_nt(p.o_b + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += pb * E::to_f32((uint16_t)(vb[i] & 0xffffu));
        acc[2 * i + 1] += pb * E::to_f32((uint16_t)(vb[i] >> 16));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = E::pack2(acc[2 * i], acc[2 * i + 1]);
    lse_out = big + fast_log2(tot) * kLn2;
  }
  if (ATTN_IN_RANGE(p.o + off, 16, p.o, (size_t)p.rows * kD * 2, kSiteMlseO)) store16_nt(p.o + off, out);
  if (p.lse != nullptr && c == 0 && ATTN_IN_RANGE(p.lse + row, 4, p.lse, (size_t)p.rows * 4, kSiteMlseLse))
    p.lse[row] = lse_out;
}

}  // namespace

ATTN_DEFINE_CHECK_READER(merge_lse)

hipError_t merge_lse(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o,
                     float* lse, int rows, int dtype, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  MergeLseParams p;
  p.o_a = static_cast<const uint16_t*>(o_a);
  p.lse_a = lse_a;
  p.o_b = static_cast<const uint16_t*>(o_b);
  p.lse_b = lse_b;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.rows = rows;
  const dim3 grid((unsigned)((rows + kRowsPerWg - 1) / kRowsPerWg));
  if (dtype == ATTN_DTYPE_BF16)
    hipLaunchKernelGGL(merge_lse_kernel<ATTN_DTYPE_BF16>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_lse_kernel<ATTN_DTYPE_F16>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
