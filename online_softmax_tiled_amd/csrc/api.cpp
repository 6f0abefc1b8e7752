// C ABI of libattn.so: argument validation, error reporting and dispatch to
// the gfx950 kernels. Every argument is checked before anything is launched;
// errors come back as codes with a per-thread message, never as exceptions
// or aborts. The conditions the pages treat as hard errors (the head count
// must be a multiple of the KV head count and the head size must be one the
// kernel was built for, "Decode attention: FlashDecoding, split-K, paged
// kernels", section "The kernel vLLM deleted"; kernel block sizes are
// multiples of 16, same page, paged addressing and section "Kernel block
// size vs allocator block size") are rejected here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "attn.h"

namespace attn {
hipError_t prefill_fwd(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                       const uint8_t* row_mask, void* o, float* lse, int B, int h, int h_kv,
                       int T_q, int T_k, int dtype, float scale, int causal, hipStream_t stream);
hipError_t decode_split(const void* q, const void* k, const void* v, const int32_t* block_table,
                        int max_pages, int page_size, int num_pages, const int32_t* seq_lens,
                        int s_max, int B, int h, int h_kv, int chunk_keys, int max_splits,
                        int dtype, float scale, float* part_o, float* part_m, float* part_l,
                        hipStream_t stream);
hipError_t decode_split_fp8kv(const void* q, const void* k, const void* v, const int32_t* block_table,
                             int max_pages, int page_size, int num_pages, const int32_t* seq_lens, int s_max,
                             int B, int h, int h_kv, int chunk_keys, int max_splits, int dtype, float scale,
                             float k_scale, float v_scale, float* part_o, float* part_m, float* part_l,
                             hipStream_t stream);
hipError_t decode_split_rows(const void* q, const void* k, const void* v, const int32_t* block_table,
                             int max_pages, int page_shift, int num_pages, const int32_t* seq_lens, int s_max,
                             int B, int h, int h_kv, int chunk_keys, int max_splits, int dtype, float scale,
                             float* part_o, float* part_m, float* part_l, hipStream_t stream, bool kv8,
                             float k_scale, float v_scale);
bool decode_rows_fp8_supported(int g, bool paged, int num_pages, int h_kv, int page_shift);
hipError_t merge_states(const float* part_o, const float* part_m, const float* part_l,
                        const int32_t* seq_lens, int chunk_keys, int B, int h, int max_splits,
                        void* o, float* lse, int dtype, hipStream_t stream);
hipError_t paged_gather(const void* pool, const int32_t* block_table, const int32_t* seq_lens,
                        int B, int h_kv, int page_size, int max_pages, int num_pages, int s_max,
                        void* out, hipStream_t stream);
hipError_t prefill_paged(const void* q, const int32_t* cu_seqlens_q, int max_q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table, const int32_t* seq_lens_k,
                         const int32_t* seq_lens_k_host, int B, int h, int h_kv, int page_shift, int max_pages,
                         int num_pages, void* o, float* lse, int dtype, float scale, int causal,
                         hipStream_t stream);
hipError_t merge_lse(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o,
                     float* lse, int rows, int dtype, hipStream_t stream);
int decode_plan(int B, const int32_t* seq_lens, int units_per_split, int wgs_per_cu, int num_cus, int32_t* chunk_keys,
                int32_t* max_splits);
hipError_t stream_read(const void* src, uint64_t bytes, int chunks, uint32_t* out, hipStream_t stream);
size_t decode_scratch_bytes();
#ifdef ATTN_DEVICE_CHECKS
hipError_t check_read_decode(uint32_t* hits);
hipError_t check_read_prefill(uint32_t* hits);
hipError_t check_read_merge(uint32_t* hits);
hipError_t check_read_merge_lse(uint32_t* hits);
hipError_t check_read_gather(uint32_t* hits);
hipError_t check_read_stream(uint32_t* hits);
hipError_t check_clear_decode();
hipError_t check_clear_prefill();
hipError_t check_clear_merge();
hipError_t check_clear_merge_lse();
hipError_t check_clear_gather();
hipError_t check_clear_stream();
hipError_t check_selftest(const void* base, hipStream_t stream);
#endif
hipError_t decode_scratch(void** ptr);
}  // namespace attn

namespace {

constexpr int kHeadDim = 128;
constexpr int kMaxGroup = 256;  // decode: query heads per KV head
// Decode groups of up to kRowsMinGroup - 1 heads use the split kernel of
// decode.hip (the heads as the 16 columns of its MFMA); larger groups use the
// prefill kernel with the heads as rows (32 per wave), which runs one
// workgroup per CU and is planned at one workgroup of work per CU. Measured
// on 268-537 MB of K+V (split + merge, contiguous / 16-token pages): g = 128
// 114 / 120 us against 366-429 us in blocks of 16 heads; g = 32 101 / 115 us
// against 148-160; g = 24 100 / 119 us against 143-144.
constexpr int kRowsMinGroup = 17;
constexpr int kRowsWgsPerCu = 1;

// log2 of a power of two, else -1.
int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}
constexpr int kMaxSeq = 1 << 23;  // keys or queries per (batch, head); decode: keys per sequence

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ATTN_OK;
}

int from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

#define REQUIRE(cond, code, ...)          \
  do {                                    \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

int check_common(const char* fn, int dtype, int d_h) {
  REQUIRE(dtype == ATTN_DTYPE_F16 || dtype == ATTN_DTYPE_BF16, ATTN_ERR_UNSUPPORTED,
          "%s: dtype %d is not supported (0 = f16, 1 = bf16)", fn, dtype);
  REQUIRE(d_h == kHeadDim, ATTN_ERR_UNSUPPORTED, "%s: head size %d is not supported (only %d)", fn, d_h,
          kHeadDim);
  return ATTN_OK;
}

int check_heads(const char* fn, int h, int h_kv) {
  REQUIRE(h > 0 && h_kv > 0, ATTN_ERR_INVALID, "%s: head counts must be positive (h=%d, h_kv=%d)", fn, h, h_kv);
  REQUIRE(h % h_kv == 0, ATTN_ERR_INVALID, "%s: h=%d is not a multiple of h_kv=%d", fn, h, h_kv);
  return ATTN_OK;
}

int check_scale(const char* fn, float scale) {
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_ERR_INVALID, "%s: scale must be finite and > 0 (got %g)", fn,
          (double)scale);
  return ATTN_OK;
}

// Arguments of a split-KV decode stage 1 (attn_decode_split, attn_decode).
int check_decode(const char* fn, const void* q, const void* k, const void* v, const int32_t* block_table,
                 int max_pages, int page_size, int num_pages, const int32_t* seq_lens, int s_max, int B, int h,
                 int h_kv, int d_h, int chunk_keys, int max_splits, int dtype, float scale) {
  if (int e = check_common(fn, dtype, d_h)) return e;
  if (int e = check_heads(fn, h, h_kv)) return e;
  if (int e = check_scale(fn, scale)) return e;
  REQUIRE(h / h_kv <= kMaxGroup, ATTN_ERR_UNSUPPORTED, "%s: %d query heads per KV head (at most %d supported)",
          fn, h / h_kv, kMaxGroup);
  REQUIRE((long)max_splits * h_kv * B < (1L << 31), ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  REQUIRE(B >= 0, ATTN_ERR_INVALID, "%s: negative batch %d", fn, B);
  REQUIRE(chunk_keys > 0 && chunk_keys % 16 == 0, ATTN_ERR_INVALID,
          "%s: chunk_keys must be a positive multiple of 16 (got %d)", fn, chunk_keys);
  REQUIRE(max_splits >= 1 && max_splits <= 65535, ATTN_ERR_INVALID, "%s: max_splits must be in [1, 65535] (got %d)",
          fn, max_splits);
  REQUIRE(h_kv <= 65535 && B <= 65535, ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  if (block_table) {
    REQUIRE(page_size > 0 && page_size % 16 == 0, ATTN_ERR_UNSUPPORTED,
            "%s: page_size must be a positive multiple of 16 (got %d)", fn, page_size);
    REQUIRE(max_pages > 0 && num_pages > 0, ATTN_ERR_INVALID, "%s: max_pages and num_pages must be positive", fn);
    REQUIRE((long)max_pages * page_size <= kMaxSeq, ATTN_ERR_UNSUPPORTED,
            "%s: max_pages * page_size = %ld keys (at most %d supported)", fn, (long)max_pages * page_size, kMaxSeq);
  } else {
    REQUIRE(s_max >= 0, ATTN_ERR_INVALID, "%s: negative s_max %d", fn, s_max);
    REQUIRE(s_max <= kMaxSeq, ATTN_ERR_UNSUPPORTED, "%s: s_max = %d keys (at most %d supported)", fn, s_max, kMaxSeq);
  }
  if (B == 0) return ATTN_OK;
  REQUIRE(q && seq_lens, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  // Contiguous K/V with s_max = 0 hold no key (every sequence is empty), so
  // they may be NULL; a paged pool always holds num_pages > 0 pages.
  REQUIRE((k && v) || (!block_table && s_max == 0), ATTN_ERR_INVALID, "%s: k and v must not be NULL", fn);
  return ATTN_OK;
}

// The per-tensor scales of 8-bit K/V.
int check_kv_scales(const char* fn, float k_scale, float v_scale) {
  REQUIRE(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f, ATTN_ERR_INVALID,
          "%s: k_scale and v_scale must be finite and > 0 (got %g, %g)", fn, (double)k_scale, (double)v_scale);
  return ATTN_OK;
}

// Stage 1 on the kernel the group size selects.
hipError_t launch_split(const void* q, const void* k, const void* v, const int32_t* block_table, int max_pages,
                        int page_size, int num_pages, const int32_t* seq_lens, int s_max, int B, int h, int h_kv,
                        int chunk_keys, int max_splits, int dtype, float scale, float* part_o, float* part_m,
                        float* part_l, hipStream_t stream) {
  const int shift = block_table ? log2_exact(page_size) : 0;
  if (h / h_kv >= kRowsMinGroup && shift >= 0)
    return attn::decode_split_rows(q, k, v, block_table, max_pages, shift, num_pages, seq_lens, s_max, B, h, h_kv,
                                   chunk_keys, max_splits, dtype, scale, part_o, part_m, part_l, stream, false, 1.f,
                                   1.f);
  return attn::decode_split(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                            chunk_keys, max_splits, dtype, scale, part_o, part_m, part_l, stream);
}

// Stage 1 over 8-bit K/V: the heads as rows for 17-128 heads per KV head
// (power-of-two pages, pools that 32-bit offsets address), else blocks of 16
// heads.
hipError_t launch_split_fp8(const void* q, const void* k, const void* v, const int32_t* block_table, int max_pages,
                            int page_size, int num_pages, const int32_t* seq_lens, int s_max, int B, int h, int h_kv,
                            int chunk_keys, int max_splits, int dtype, float scale, float k_scale, float v_scale,
                            float* part_o, float* part_m, float* part_l, hipStream_t stream) {
  const int shift = block_table ? log2_exact(page_size) : 0;
  if (h / h_kv >= kRowsMinGroup && shift >= 0 &&
      attn::decode_rows_fp8_supported(h / h_kv, block_table != nullptr, num_pages, h_kv, shift))
    return attn::decode_split_rows(q, k, v, block_table, max_pages, shift, num_pages, seq_lens, s_max, B, h, h_kv,
                                   chunk_keys, max_splits, dtype, scale, part_o, part_m, part_l, stream, true,
                                   k_scale, v_scale);
  return attn::decode_split_fp8kv(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                                  chunk_keys, max_splits, dtype, scale, k_scale, v_scale, part_o, part_m, part_l,
                                  stream);
}

}  // namespace

extern "C" {

int attn_prefill_fwd(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                     const uint8_t* row_mask, void* o, float* lse, int B, int h, int h_kv, int T_q,
                     int T_k, int d_h, int dtype, float scale, int causal, void* stream) {
  const char* fn = "attn_prefill_fwd";
  if (int e = check_common(fn, dtype, d_h)) return e;
  if (int e = check_heads(fn, h, h_kv)) return e;
  if (int e = check_scale(fn, scale)) return e;
  REQUIRE(B >= 0 && T_q >= 0 && T_k >= 0, ATTN_ERR_INVALID, "%s: negative size (B=%d, T_q=%d, T_k=%d)", fn, B,
          T_q, T_k);
  REQUIRE(!causal || T_q <= T_k, ATTN_ERR_UNSUPPORTED, "%s: causal attention needs T_q <= T_k (T_q=%d, T_k=%d)",
          fn, T_q, T_k);
  // Tiles are addressed with 32-bit byte offsets inside one (batch, head) slab.
  REQUIRE(T_q <= kMaxSeq && T_k <= kMaxSeq, ATTN_ERR_UNSUPPORTED, "%s: sequence longer than %d (T_q=%d, T_k=%d)", fn,
          kMaxSeq, T_q, T_k);
  const long rows = (long)B * h * T_q;
  REQUIRE(rows * kHeadDim < (1L << 40), ATTN_ERR_INVALID, "%s: problem too large", fn);
  // (batch, head) pairs are numbered in 32-bit ints on the device.
  REQUIRE((long)B * h < (1L << 31), ATTN_ERR_UNSUPPORTED, "%s: B * h = %ld too large", fn, (long)B * h);
  if (rows == 0) return ok();
  REQUIRE(q && o, ATTN_ERR_INVALID, "%s: q and o must not be NULL", fn);
  REQUIRE(T_k == 0 || (k && v), ATTN_ERR_INVALID, "%s: k and v must not be NULL", fn);
  return from_hip(attn::prefill_fwd(q, k, v, key_mask, row_mask, o, lse, B, h, h_kv, T_q, T_k, dtype, scale,
                                    causal, static_cast<hipStream_t>(stream)),
                  fn);
}

int attn_prefill_paged(const void* q, const int32_t* cu_seqlens_q, int max_q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, const int32_t* seq_lens_k,
                       const int32_t* seq_lens_k_host, int B, int h,
                       int h_kv, int d_h, int page_size, int max_pages, int num_pages, int dtype, float scale,
                       int causal, void* o, float* lse, void* stream) {
  const char* fn = "attn_prefill_paged";
  if (int e = check_common(fn, dtype, d_h)) return e;
  if (int e = check_heads(fn, h, h_kv)) return e;
  if (int e = check_scale(fn, scale)) return e;
  REQUIRE(B >= 0 && max_q >= 0, ATTN_ERR_INVALID, "%s: negative size (B=%d, max_q=%d)", fn, B, max_q);
  REQUIRE(page_size >= 16 && page_size <= (1 << 16) && (page_size & (page_size - 1)) == 0, ATTN_ERR_UNSUPPORTED,
          "%s: page_size must be a power of two in [16, 65536] (got %d)", fn, page_size);
  REQUIRE(max_pages > 0 && num_pages > 0, ATTN_ERR_INVALID, "%s: max_pages and num_pages must be positive", fn);
  REQUIRE((long)max_pages * page_size <= kMaxSeq, ATTN_ERR_UNSUPPORTED, "%s: more than %d keys per sequence", fn,
          kMaxSeq);
  // Q rows of one head are addressed with 32-bit byte offsets (stride h * d).
  REQUIRE((long)max_q * h * kHeadDim * 2 < (1L << 32), ATTN_ERR_UNSUPPORTED, "%s: max_q * h too large", fn);
  const long n_grp = ((long)(h / h_kv) * ((max_q + 31) / 32) + 7) / 8;
  REQUIRE(n_grp * B * h_kv < (1L << 31), ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  if (B == 0 || max_q == 0) return ok();
  REQUIRE(q && cu_seqlens_q && k_pool && v_pool && block_table && seq_lens_k && o, ATTN_ERR_INVALID,
          "%s: a required pointer is NULL", fn);
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  return from_hip(attn::prefill_paged(q, cu_seqlens_q, max_q, k_pool, v_pool, block_table, seq_lens_k,
                                      seq_lens_k_host, B, h, h_kv,
                                      shift, max_pages, num_pages, o, lse, dtype, scale, causal,
                                      static_cast<hipStream_t>(stream)),
                  fn);
}

int attn_decode_plan(int B, const int32_t* seq_lens_host, int h, int h_kv, int d_h, int num_cus,
                     int32_t* chunk_keys, int32_t* max_splits) {
  const char* fn = "attn_decode_plan";
  if (int e = check_heads(fn, h, h_kv)) return e;
  REQUIRE(d_h == kHeadDim, ATTN_ERR_UNSUPPORTED, "%s: head size %d is not supported (only %d)", fn, d_h,
          kHeadDim);
  REQUIRE(B >= 0, ATTN_ERR_INVALID, "%s: negative batch %d", fn, B);
  REQUIRE(num_cus > 0, ATTN_ERR_INVALID, "%s: num_cus must be positive (got %d)", fn, num_cus);
  REQUIRE(chunk_keys && max_splits, ATTN_ERR_INVALID, "%s: output pointers must not be NULL", fn);
  REQUIRE(B == 0 || seq_lens_host, ATTN_ERR_INVALID, "%s: seq_lens_host must not be NULL", fn);
  for (int b = 0; b < B; ++b)
    REQUIRE(seq_lens_host[b] >= 0, ATTN_ERR_INVALID, "%s: seq_lens[%d] = %d is negative", fn, b, seq_lens_host[b]);
  // One workgroup per KV head and split: the small decode workgroups run
  // several per CU, the row kernel's one per CU.
  const bool rows = h / h_kv >= kRowsMinGroup;
  attn::decode_plan(B, seq_lens_host, h_kv, rows ? kRowsWgsPerCu : 12, num_cus, chunk_keys, max_splits);
  return ok();
}

int attn_decode_plan_fixed(int B, const int32_t* seq_lens_host, int split_keys, int32_t* chunk_keys,
                           int32_t* max_splits) {
  const char* fn = "attn_decode_plan_fixed";
  REQUIRE(B >= 0, ATTN_ERR_INVALID, "%s: negative batch %d", fn, B);
  REQUIRE(split_keys > 0 && split_keys % 16 == 0, ATTN_ERR_INVALID,
          "%s: split_keys must be a positive multiple of 16 (got %d)", fn, split_keys);
  REQUIRE(chunk_keys && max_splits, ATTN_ERR_INVALID, "%s: output pointers must not be NULL", fn);
  REQUIRE(B == 0 || seq_lens_host, ATTN_ERR_INVALID, "%s: seq_lens_host must not be NULL", fn);
  int s_max = 0;
  for (int b = 0; b < B; ++b) {
    REQUIRE(seq_lens_host[b] >= 0, ATTN_ERR_INVALID, "%s: seq_lens[%d] = %d is negative", fn, b, seq_lens_host[b]);
    s_max = seq_lens_host[b] > s_max ? seq_lens_host[b] : s_max;
  }
  // A sequence's split count depends on its own length only: the splits are
  // [i * split_keys, (i + 1) * split_keys), and the grid covers the longest.
  const long splits = s_max == 0 ? 1 : ((long)s_max + split_keys - 1) / split_keys;
  REQUIRE(splits <= 65535, ATTN_ERR_UNSUPPORTED, "%s: %ld splits of %d keys (at most 65535 supported)", fn, splits,
          split_keys);
  *chunk_keys = split_keys;
  *max_splits = (int32_t)splits;
  return ok();
}

int attn_decode_split(const void* q, const void* k, const void* v, const int32_t* block_table, int max_pages,
                      int page_size, int num_pages, const int32_t* seq_lens, int s_max, int B, int h, int h_kv,
                      int d_h, int chunk_keys, int max_splits, int dtype, float scale, float* part_o,
                      float* part_m, float* part_l, void* stream) {
  const char* fn = "attn_decode_split";
  if (int e = check_decode(fn, q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                           d_h, chunk_keys, max_splits, dtype, scale))
    return e;
  if (B == 0) return ok();
  REQUIRE(part_o && part_m && part_l, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  return from_hip(launch_split(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                               chunk_keys, max_splits, dtype, scale, part_o, part_m, part_l,
                               static_cast<hipStream_t>(stream)),
                  fn);
}

int attn_decode_split_fp8kv(const void* q, const void* k, const void* v, const int32_t* block_table,
                             int max_pages, int page_size, int num_pages, const int32_t* seq_lens, int s_max, int B,
                             int h, int h_kv, int d_h, int chunk_keys, int max_splits, int dtype, float scale,
                             float k_scale, float v_scale, float* part_o, float* part_m, float* part_l,
                             void* stream) {
  const char* fn = "attn_decode_split_fp8kv";
  if (int e = check_decode(fn, q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                           d_h, chunk_keys, max_splits, dtype, scale))
    return e;
  if (int e = check_kv_scales(fn, k_scale, v_scale)) return e;
  if (B == 0) return ok();
  REQUIRE(part_o && part_m && part_l, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  return from_hip(launch_split_fp8(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                                   chunk_keys, max_splits, dtype, scale, k_scale, v_scale, part_o, part_m, part_l,
                                   static_cast<hipStream_t>(stream)),
                  fn);
}

int attn_decode_fp8kv(const void* q, const void* k, const void* v, const int32_t* block_table, int max_pages,
                      int page_size, int num_pages, const int32_t* seq_lens, int s_max, int B, int h, int h_kv,
                      int d_h, int chunk_keys, int max_splits, int dtype, float scale, float k_scale,
                      float v_scale, float* part_o, float* part_m, float* part_l, void* o, float* lse,
                      void* stream) {
  const char* fn = "attn_decode_fp8kv";
  if (int e = check_decode(fn, q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                           d_h, chunk_keys, max_splits, dtype, scale))
    return e;
  if (int e = check_kv_scales(fn, k_scale, v_scale)) return e;
  if (B == 0) return ok();
  REQUIRE(part_o && part_m && part_l && o, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  REQUIRE((long)B * h < (1L << 31), ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_split_fp8(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h,
                                       h_kv, chunk_keys, max_splits, dtype, scale, k_scale, v_scale, part_o, part_m,
                                       part_l, s);
  if (e != hipSuccess) return from_hip(e, fn);
  return from_hip(attn::merge_states(part_o, part_m, part_l, seq_lens, chunk_keys, B, h, max_splits, o, lse, dtype, s),
                  fn);
}

int attn_decode(const void* q, const void* k, const void* v, const int32_t* block_table, int max_pages,
                int page_size, int num_pages, const int32_t* seq_lens, int s_max, int B, int h, int h_kv, int d_h,
                int chunk_keys, int max_splits, int dtype, float scale, float* part_o, float* part_m,
                float* part_l, void* o, float* lse, void* stream) {
  const char* fn = "attn_decode";
  if (int e = check_decode(fn, q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                           d_h, chunk_keys, max_splits, dtype, scale))
    return e;
  if (B == 0) return ok();
  REQUIRE(part_o && part_m && part_l && o, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  REQUIRE((long)B * h < (1L << 31), ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_split(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h,
                                    h_kv, chunk_keys, max_splits, dtype, scale, part_o, part_m, part_l, s);
  if (e != hipSuccess) return from_hip(e, fn);
  return from_hip(attn::merge_states(part_o, part_m, part_l, seq_lens, chunk_keys, B, h, max_splits, o, lse, dtype, s),
                  fn);
}

int attn_decode_noalloc(const void* q, const void* k, const void* v, const int32_t* block_table, int max_pages,
                        int page_size, int num_pages, const int32_t* seq_lens, int s_max, int B, int h, int h_kv,
                        int d_h, int chunk_keys, int max_splits, int dtype, float scale, void* o, float* lse,
                        void* stream) {
  const char* fn = "attn_decode_noalloc";
  if (int e = check_decode(fn, q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h, h_kv,
                           d_h, chunk_keys, max_splits, dtype, scale))
    return e;
  if (B == 0) return ok();
  REQUIRE(o, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  REQUIRE((long)B * h < (1L << 31), ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  // partial states: part_o [B, h, S, d], then part_m and part_l [B, h, S]
  const size_t rows = (size_t)B * h * max_splits;
  const size_t need = rows * (kHeadDim + 2) * sizeof(float);
  REQUIRE(need <= attn::decode_scratch_bytes(), ATTN_ERR_UNSUPPORTED,
          "%s: B * h * max_splits = %zu partial states need %zu bytes; the device scratch holds %zu", fn, rows, need,
          attn::decode_scratch_bytes());
  void* base = nullptr;
  const hipError_t es = attn::decode_scratch(&base);
  if (es != hipSuccess) return from_hip(es, fn);
  float* part_o = static_cast<float*>(base);
  float* part_m = part_o + rows * kHeadDim;
  float* part_l = part_m + rows;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_split(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h,
                                    h_kv, chunk_keys, max_splits, dtype, scale, part_o, part_m, part_l, s);
  if (e != hipSuccess) return from_hip(e, fn);
  return from_hip(attn::merge_states(part_o, part_m, part_l, seq_lens, chunk_keys, B, h, max_splits, o, lse, dtype, s),
                  fn);
}

int attn_merge_states(const float* part_o, const float* part_m, const float* part_l, const int32_t* seq_lens,
                      int chunk_keys, int B, int h, int max_splits, int d_h, void* o, float* lse, int dtype,
                      void* stream) {
  const char* fn = "attn_merge_states";
  if (int e = check_common(fn, dtype, d_h)) return e;
  REQUIRE(B >= 0 && h > 0, ATTN_ERR_INVALID, "%s: bad sizes (B=%d, h=%d)", fn, B, h);
  REQUIRE(chunk_keys > 0, ATTN_ERR_INVALID, "%s: chunk_keys must be positive (got %d)", fn, chunk_keys);
  REQUIRE(max_splits >= 1, ATTN_ERR_INVALID, "%s: max_splits must be >= 1 (got %d)", fn, max_splits);
  if (B == 0) return ok();
  REQUIRE((long)B * h < (1L << 31), ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  REQUIRE(part_o && part_m && part_l && seq_lens && o, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  return from_hip(attn::merge_states(part_o, part_m, part_l, seq_lens, chunk_keys, B, h, max_splits, o, lse, dtype,
                                     static_cast<hipStream_t>(stream)),
                  fn);
}

int attn_merge_lse(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, int rows, int d_h,
                   void* o, float* lse, int dtype, void* stream) {
  const char* fn = "attn_merge_lse";
  if (int e = check_common(fn, dtype, d_h)) return e;
  REQUIRE(rows >= 0, ATTN_ERR_INVALID, "%s: rows must be non-negative (got %d)", fn, rows);
  if (rows == 0) return ok();
  REQUIRE(o_a && lse_a && o_b && lse_b && o, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  return from_hip(attn::merge_lse(o_a, lse_a, o_b, lse_b, o, lse, rows, dtype, static_cast<hipStream_t>(stream)), fn);
}

int attn_paged_gather(const void* pool, const int32_t* block_table, const int32_t* seq_lens, int B, int h_kv,
                      int d_h, int page_size, int max_pages, int num_pages, int s_max, int dtype, void* out,
                      void* stream) {
  const char* fn = "attn_paged_gather";
  if (int e = check_common(fn, dtype, d_h)) return e;
  REQUIRE(B >= 0 && h_kv > 0 && s_max >= 0, ATTN_ERR_INVALID, "%s: bad sizes (B=%d, h_kv=%d, s_max=%d)", fn, B,
          h_kv, s_max);
  REQUIRE(page_size > 0 && max_pages > 0 && num_pages > 0, ATTN_ERR_INVALID,
          "%s: page_size, max_pages and num_pages must be positive", fn);
  REQUIRE(B <= 65535, ATTN_ERR_UNSUPPORTED, "%s: grid too large", fn);
  REQUIRE((long)max_pages * page_size < (1L << 31), ATTN_ERR_UNSUPPORTED,
          "%s: max_pages * page_size = %ld keys (at most 2^31 - 1 supported)", fn, (long)max_pages * page_size);
  if (B == 0 || s_max == 0) return ok();
  REQUIRE(pool && block_table && seq_lens && out, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  return from_hip(attn::paged_gather(pool, block_table, seq_lens, B, h_kv, page_size, max_pages, num_pages, s_max,
                                     out, static_cast<hipStream_t>(stream)),
                  fn);
}

int attn_stream_read(const void* src, uint64_t bytes, int chunks, uint32_t* out, void* stream) {
  const char* fn = "attn_stream_read";
  REQUIRE(chunks >= 1 && chunks <= 65536, ATTN_ERR_INVALID, "%s: chunks must be in [1, 65536] (got %d)", fn, chunks);
  REQUIRE(bytes % 16 == 0, ATTN_ERR_INVALID, "%s: bytes must be a multiple of 16", fn);
  REQUIRE(src && out, ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
  REQUIRE(((uintptr_t)src & 15) == 0, ATTN_ERR_INVALID, "%s: src must be 16-byte aligned", fn);
  return from_hip(attn::stream_read(src, bytes, chunks, out, static_cast<hipStream_t>(stream)), fn);
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

const char* attn_version(void) {
#ifdef ATTN_DEVICE_CHECKS
  return "libattn 0.1 (gfx950, device bounds checks)";
#else
  return "libattn 0.1 (gfx950)";
#endif
}

int attn_check_report(uint32_t* hits, int n_sites) {
  const char* fn = "attn_check_report";
#ifdef ATTN_DEVICE_CHECKS
  REQUIRE(hits != nullptr && n_sites >= ATTN_CHECK_SITES, ATTN_ERR_INVALID, "%s: need room for %d sites", fn,
          (int)ATTN_CHECK_SITES);
  hipError_t (*readers[])(uint32_t*) = {attn::check_read_decode, attn::check_read_prefill, attn::check_read_merge,
                                        attn::check_read_merge_lse, attn::check_read_gather, attn::check_read_stream};
  for (int i = 0; i < ATTN_CHECK_SITES; ++i) hits[i] = 0u;
  for (auto rd : readers) {
    uint32_t part[ATTN_CHECK_SITES];
    const hipError_t e = rd(part);
    if (e != hipSuccess) return from_hip(e, fn);
    for (int i = 0; i < ATTN_CHECK_SITES; ++i) hits[i] |= part[i];
  }
  return ok();
#else
  (void)hits;
  (void)n_sites;
  return fail(ATTN_ERR_UNSUPPORTED, "%s: this library was built without device bounds checks", fn);
#endif
}

int attn_check_selftest(const void* base, void* stream) {
  const char* fn = "attn_check_selftest";
#ifdef ATTN_DEVICE_CHECKS
  REQUIRE(base != nullptr, ATTN_ERR_INVALID, "%s: base must not be NULL", fn);
  return from_hip(attn::check_selftest(base, static_cast<hipStream_t>(stream)), fn);
#else
  (void)base;
  (void)stream;
  return fail(ATTN_ERR_UNSUPPORTED, "%s: this library was built without device bounds checks", fn);
#endif
}

int attn_check_clear(void) {
  const char* fn = "attn_check_clear";
#ifdef ATTN_DEVICE_CHECKS
  hipError_t (*clears[])() = {attn::check_clear_decode, attn::check_clear_prefill, attn::check_clear_merge,
                              attn::check_clear_merge_lse, attn::check_clear_gather, attn::check_clear_stream};
  for (auto cl : clears) {
    const hipError_t e = cl();
    if (e != hipSuccess) return from_hip(e, fn);
  }
  return ok();
#else
  return fail(ATTN_ERR_UNSUPPORTED, "%s: this library was built without device bounds checks", fn);
#endif
}

}  // extern "C"
