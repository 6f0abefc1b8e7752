// Shared device helpers for the gfx950 (CDNA4) attention kernels: element
// types, MFMA wrappers, packed conversions, fp32 exp2/log2 on the hardware
// transcendental unit, and the error plumbing of the host side.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32). The
// kernels keep logits in base-2 units (x * scale * log2 e) so that one
// multiply-add and one v_exp_f32 give exp(x - m); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Per-dtype operations. DT = ATTN_DTYPE_F16 or ATTN_DTYPE_BF16. Operands are
// passed around as raw 16-byte vectors (u32x4 = 8 elements).
template <int DT>
struct Elem;

template <>
struct Elem<ATTN_DTYPE_BF16> {
  // D(32x32 fp32) += A(32x16) * B(16x32); A lane l holds row l%32, k in
  // [8*(l/32), 8*(l/32)+8); B lane l holds column l%32, same k range.
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // D(16x16 fp32) += A(16x32) * B(32x16); A lane l holds row l%16, k in
  // [8*(l/16), 8*(l/16)+8); B lane l holds column l%16, same k range.
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two fp32 -> two bf16 (round to nearest even), lo in bits [15:0].
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  static __device__ __forceinline__ float to_f32(uint16_t x) {
    return __builtin_bit_cast(float, (uint32_t)x << 16);
  }
  // acc + lo + hi of a packed pair, in fp32 (v_dot2 with a (1, 1) operand).
  static __device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                           acc, false);
  }
};

template <>
struct Elem<ATTN_DTYPE_F16> {
  static __device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ float to_f32(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
  static __device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), __builtin_bit_cast(f16x2, 0x3C003C00u), acc,
                                  false);
  }
};

// A pair of bf16 values (lo in bits [15:0]) as a pair of fp16 values,
// rounded to nearest. Every bf16 value of magnitude in [2^-14, 65536) is an
// fp16 value (fp16 has more significand bits and covers that exponent range),
// so these convert exactly; smaller ones land on the fp16 subnormal grid
// (absolute error at most 2^-25), and magnitudes of 65536 or more overflow to
// +-inf (the largest bf16 value below 65536 is 65280, which fp16 holds), so
// that a product that uses one comes out inf or NaN.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  const float lo = __builtin_bit_cast(float, x << 16);
  const float hi = __builtin_bit_cast(float, x & 0xffff0000u);
  return Elem<ATTN_DTYPE_F16>::pack2(lo, hi);
}

// True when any of the 64 accumulator values is inf or NaN (exponent field
// all ones), tested on the bits so that no floating-point assumption about
// NaN can remove the test. Each element is copied to a scalar before the
// bit cast: this compiler lowers a bit cast of a subscripted vector element
// as a load from the vector's first element, whatever the subscript.
__device__ __forceinline__ bool any_nonfinite(const f32x16 (&acc)[4]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float x = acc[i][e];
      m = max(m, __builtin_bit_cast(uint32_t, x) & 0x7fffffffu);
    }
  return m >= 0x7f800000u;
}

// Eight E4M3 codes (two words, code e in byte e % 4 of word e / 4) as eight
// 16-bit operands of type DT, with gfx950's packed fp8 conversion at scale
// 1, which is exact (every E4M3 value is an fp16 and a bf16 value); element
// e lands in half e % 2 of word e / 2, as a 16-bit load would put it.
template <int DT>
__device__ __forceinline__ u32x4 cvt8(u32x2 x) {
  // (the half-word select of the conversion is an immediate)
  if constexpr (DT == ATTN_DTYPE_BF16)
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true))};
  else
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.0f, true))};
}

// Word sel (0: codes 0-1, 1: codes 2-3) of cvt8 of one word.
template <int DT>
__device__ __forceinline__ uint32_t cvt8w(uint32_t w, int sel) {
  if constexpr (DT == ATTN_DTYPE_BF16)
    return sel ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
               : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  else
    return sel ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
               : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}

// Byte select of v_perm_b32: result byte i = byte sel[i] of {hi:lo} (0-3 lo).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// (low half of a, low half of b) and (high half of a, high half of b).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// The values of x on lanes l % 32 and l % 32 + 32, on every lane l: gfx950's
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with
// the lower 32 lanes of its second, a vector-ALU exchange with no LDS round
// trip. Written as assembly with both operands read-write: with the compiler
// builtin and the same value in both operands, this compiler folds a
// combination of the two results into the first result alone (a kernel
// returning their sum emits v_add_f32 v1, v1, v1). The s_nop gives the two
// wait states between a vector write of an operand and the swap reading it.
// Not volatile: the swap is a pure function of its operands, and a volatile
// statement counts as a possible memory write, after which the compiler no
// longer reads read-only tables (the decode's block table) with scalar loads.
__device__ __forceinline__ void swap_halves(float x, float& lo, float& hi) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second; with x in both, lo holds x of row 2j and hi x
// of row 2j + 1 in every lane of the row pair j (same position in the row).
// Assembly for the same reasons as above.
__device__ __forceinline__ void swap_rows16(float x, float& lo, float& hi) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
// Max / sum of x over lanes l and l ^ 32 (the two halves of a wave64); both
// lanes of a pair get the same bits (the lower lane's value first).
__device__ __forceinline__ float max_halves(float x) {
  float lo, hi;
  swap_halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float x) {
  float lo, hi;
  swap_halves(x, lo, hi);
  return lo + hi;
}

// Debug build with device-side bounds checks (-DATTN_DEVICE_CHECKS,
// libattn_checked.so). Every raw global access (one not made through a
// range-checked buffer resource), and every buffer range a kernel builds, is
// first tested against the extent of its tensor, computed from the kernel's
// own parameters. A failing access is not made (a load gives zeros, a store
// is dropped) and the flag of its site is set with a plain vector store; the
// host reads the flags back (attn_check_report). In the product build the
// tests compile away. Sites are numbered across the kernel files (CheckSite).
enum CheckSite {
  kSiteDecSeqLens = 0, kSiteDecQ, kSiteDecTable, kSiteDecK16, kSiteDecV16, kSiteDecK8, kSiteDecV8, kSiteDecTable8,
  kSiteDecPartO, kSiteDecPartML,
  kSitePreLens = 16, kSitePreQ, kSitePreKV, kSitePreKeyRow, kSitePreTableRow, kSitePrePagedKV, kSitePrePartO,
  kSitePrePartML, kSitePreO, kSitePreLse, kSitePreRowMask,
  kSiteMrgLens = 32, kSiteMrgPartML, kSiteMrgPartO, kSiteMrgO, kSiteMrgLse,
  kSiteMlseIn = 40, kSiteMlseO, kSiteMlseLse,
  kSiteGthLens = 44, kSiteGthTable, kSiteGthPool, kSiteGthOut,
  kSiteStream = 48,
  kSiteSelfTestIn = 62, kSiteSelfTestOut = 63,   // attn_check_selftest
  kCheckSites = ATTN_CHECK_SITES
};
#ifdef ATTN_DEVICE_CHECKS
static __device__ uint32_t check_hits[kCheckSites];
__device__ __forceinline__ bool in_range(const void* p, size_t bytes, const void* base, size_t extent, int site) {
  const char* a = static_cast<const char*>(p);
  const char* b = static_cast<const char*>(base);
  const bool ok = a >= b && (size_t)(a - b) + bytes <= extent;
  if (!ok) check_hits[site] = 1u;
  return ok;
}
#define ATTN_IN_RANGE(p, bytes, base, extent, site) ::attn::in_range((p), (bytes), (base), (extent), (site))
// The host side of one kernel file's flags (each file has its own array).
#define ATTN_DEFINE_CHECK_READER(name)                                                        \
  hipError_t check_read_##name(uint32_t* hits) {                                              \
    return hipMemcpyFromSymbol(hits, HIP_SYMBOL(check_hits), sizeof(uint32_t) * kCheckSites); \
  }                                                                                           \
  hipError_t check_clear_##name() {                                                           \
    uint32_t z[kCheckSites] = {};                                                             \
    return hipMemcpyToSymbol(HIP_SYMBOL(check_hits), z, sizeof(z));                           \
  }
#else
#define ATTN_IN_RANGE(p, bytes, base, extent, site) true
#define ATTN_DEFINE_CHECK_READER(name)
#endif

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming load: non-temporal hint, for data read exactly once (decode K/V),
// so it does not displace reused lines from the caches.
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Buffer resource over [base, base + bytes): a raw buffer load past the end
// returns zeros instead of touching memory, so tile loads need no branches.
// Word 3 (0x00020000) is the CDNA default for untyped 32-bit data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// gfx950 transposing LDS read of four 16-bit elements. Within each group of
// 16 lanes, result element k of lane i is element i % 4 of the 8 bytes that
// lane 4k + i / 4 addresses.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming store: non-temporal hint, for output written once and not reread.
__device__ __forceinline__ void store16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

}  // namespace attn
