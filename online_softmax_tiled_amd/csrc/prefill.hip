// Prefill attention for gfx950: one pass over key tiles with the online
// softmax state (m, l, O~) held in registers; the score tile lives only in
// VGPRs ("Naive attention and the online softmax", sections (3) "The online
// recurrence" and "Extending the recurrence to the output").
//
// Work decomposition
//   A workgroup is 4 waves. Each wave owns one block of 32 query rows of one
//   query head; the 4 blocks of a workgroup belong to query heads that share
//   one KV head (row blocks are numbered query-block-major, head-minor inside
//   a GQA group), so every K/V tile staged in LDS feeds all 4 waves.
//   Workgroups are numbered with (batch, kv head) fastest so that consecutive
//   workgroups -- which the hardware deals round-robin to the 8 XCDs -- put
//   each KV head's workgroups on one XCD and its L2; the longest causal row
//   blocks are numbered first.
//
// Per 64-key tile and wave
//   S^T = K Q^T on v_mfma_f32_32x32x16 (A = K rows from LDS, B = the wave's
//   Q rows held in VGPRs for the whole kernel). In the accumulator layout
//   lane l holds query row l%32 and, for register r of 32-key block kb, key
//   kb*32 + 8*(r/4) + 4*(l/32) + r%4. A row's 64 scores thus sit in one lane
//   pair (l, l^32): the row max is an in-lane max plus one half swap.
//   Online update in base 2: c = scale*log2(e), m' = max(m, c*max s),
//   alpha = 2^(m - m'), p = 2^(c*s - m'), l = alpha*l + sum p, O~ *= alpha.
//   While a row has seen no visible key (m' = -inf) the subtracted reference
//   is 0 instead of m', so -inf - (-inf) is never formed ("Merge normalized
//   attention without averaging tile outputs", paragraph on fully masked
//   tiles).
//   O~^T += V^T P^T on the same MFMA: P^T is used straight from the score
//   registers as the B operand (rounded to the operand dtype); V^T comes
//   from LDS, where the staging threads stored V transposed with bits 2 and
//   3 of the key index swapped inside each 16-key group so that each A
//   operand is one 16-byte LDS read.
//   Masking (causal, key range, key mask) is applied only in tiles that
//   need it; tiles with no visible key for a wave are skipped.
//
// Epilogue: O = O~/l rounded to the output dtype, LSE = (m + log2 l) ln 2.
// l = 0 (no visible key) or a zero row-mask entry gives +0.0 output and
// LSE = -inf ("Merge normalized attention without averaging tile outputs",
// last paragraph).
#include "common.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kRows = 32;           // query rows per wave
constexpr int kBc = 64;             // keys per tile
constexpr int kKStr = kD + 8;       // K row stride in LDS (elements): 272 B
constexpr int kVStr = kBc + 8;      // V^T row stride in LDS (elements): 144 B
constexpr int kKElems = kBc * kKStr;
constexpr int kVElems = kD * kVStr;

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* key_mask;
  const uint8_t* row_mask;
  uint16_t* o;
  float* lse;
  int B, h, h_kv, T_q, T_k;
  int g;        // h / h_kv
  int n_rb;     // row blocks per (batch, kv head) = g * ceil(T_q / 32)
  int n_grp;    // workgroups per (batch, kv head) = ceil(n_rb / 4)
  float c;      // scale * log2(e)
};

// Position of tile key kk (0..63) inside a V^T row of LDS.
__device__ __forceinline__ int vt_pos(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <int DT, bool CAUSAL, bool KMASK>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  using E = Elem<DT>;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKElems];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kVElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query row inside the wave's block
  const int half = lane >> 5;

  const int n_bk = p.B * p.h_kv;
  const int bk = blockIdx.x % n_bk;
  const int grp = p.n_grp - 1 - (int)(blockIdx.x / n_bk);
  const int b = bk / p.h_kv;
  const int kvh = bk - b * p.h_kv;

  const int rb = grp * kWaves + wave;
  const bool wave_valid = rb < p.n_rb;
  const int qblk = rb / p.g;
  const int head = kvh * p.g + (rb - qblk * p.g);
  const int q0 = qblk * kRows;
  const int off = p.T_k - p.T_q;   // >= 0 when causal
  const int qrow = q0 + col;
  const int row_last_w = min(p.T_q - 1, q0 + kRows - 1);

  const int rb_last = min(grp * kWaves + kWaves - 1, p.n_rb - 1);
  const int row_last_wg = min(p.T_q - 1, (rb_last / p.g) * kRows + kRows - 1);
  int n_tiles = (p.T_k + kBc - 1) / kBc;
  if (CAUSAL) n_tiles = min(n_tiles, (row_last_wg + off) / kBc + 1);

  // Q rows of this wave as MFMA B operands: lane holds row col, d in
  // [16c + 8*half, 16c + 8*half + 8).
  u32x4 qf[8];
  {
    const bool ok = wave_valid && qrow < p.T_q;
    const uint16_t* qp = p.q + ((size_t)(b * p.h + head) * p.T_q + (ok ? qrow : 0)) * kD + half * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = ok ? load16(qp + c * 16) : u32x4{0, 0, 0, 0};
  }

  const size_t kv_base = (size_t)bk * p.T_k * kD;
  const uint16_t* kg = p.k + kv_base;
  const uint16_t* vg = p.v + kv_base;

  // Staging registers: K as 4 chunks of 16 B (key chunk>>4, d-chunk chunk&15),
  // V as 4 consecutive keys x 8 d for a transposed store.
  u32x4 kreg[4], vreg[4];
  const int v_kq = tid >> 4;   // 4-key group 0..15
  const int v_dg = tid & 15;   // 8-d group 0..15

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = tid + 256 * i;
      const int key = kt + (chunk >> 4);
      kreg[i] = key < p.T_k ? load16(kg + (size_t)key * kD + (chunk & 15) * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kt + v_kq * 4 + i;
      vreg[i] = key < p.T_k ? load16(vg + (size_t)key * kD + v_dg * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = tid + 256 * i;
      store16(&lds_k[buf][(chunk >> 4) * kKStr + (chunk & 15) * 8], kreg[i]);
    }
    const int pos = vt_pos(v_kq * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = v_dg * 8 + 2 * e;
      store8(&lds_v[buf][d * kVStr + pos],
             u32x2{pack_lo16(vreg[0][e], vreg[1][e]), pack_lo16(vreg[2][e], vreg[3][e])});
      store8(&lds_v[buf][(d + 1) * kVStr + pos],
             u32x2{pack_hi16(vreg[0][e], vreg[1][e]), pack_hi16(vreg[2][e], vreg[3][e])});
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;   // running max, base-2 scaled units
  float l_run = 0.f;         // this lane's share of the running sum

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int kt = j * kBc;
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(kt + kBc);

    uint64_t kbits = ~0ull;
    if (KMASK) {
      const int key = kt + lane;
      const bool on = key < p.T_k && p.key_mask[(size_t)b * p.T_k + key] != 0;
      kbits = __ballot(on);
    }
    bool skip = !wave_valid;
    if (CAUSAL) skip = skip || kt > row_last_w + off;
    if (KMASK) skip = skip || kbits == 0;

    if (!skip) {
      const uint16_t* ks = lds_k[buf];
      const uint16_t* vs = lds_v[buf];
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* kr = ks + (kb * 32 + col) * kKStr + half * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) s[kb] = E::mfma32(load16(kr + c * 16), qf[c], s[kb]);
      }

      bool need_mask = kt + kBc > p.T_k;
      if (CAUSAL) need_mask = need_mask || (kt + kBc - 1 > q0 + off);
      if (KMASK) need_mask = need_mask || (kbits != ~0ull);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            bool vis = kt + ko < p.T_k;
            if (CAUSAL) vis = vis && (kt + ko <= qrow + off);
            if (KMASK) vis = vis && ((kbits >> ko) & 1ull);
            s[kb][r] = vis ? s[kb][r] : -INFINITY;
          }
        }
      }

      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = max_halves(mx);
      const float m_new = fmaxf(m_run, mx * p.c);
      const float base = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - base);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(__builtin_fmaf(s[kb][r], p.c, -base));
          s[kb][r] = e;
          rs += e;
        }
      }
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= alpha;
      }

      // P^T as B operands: 16-key chunk cc uses registers 8*(cc%2).. of block cc/2.
      u32x4 pf[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const f32x16& sv = s[cc >> 1];
        const int r0 = (cc & 1) * 8;
        pf[cc] = u32x4{E::pack2(sv[r0 + 0], sv[r0 + 1]), E::pack2(sv[r0 + 2], sv[r0 + 3]),
                       E::pack2(sv[r0 + 4], sv[r0 + 5]), E::pack2(sv[r0 + 6], sv[r0 + 7])};
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* vr = vs + (db * 32 + col) * kVStr + half * 8;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) acc[db] = E::mfma32(load16(vr + cc * 16), pf[cc], acc[db]);
      }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_valid || qrow >= p.T_q) return;
  const float l_tot = sum_halves(l_run);
  bool empty = l_tot == 0.f;
  if (p.row_mask != nullptr) empty = empty || p.row_mask[(size_t)b * p.T_q + qrow] == 0;
  const float inv = empty ? 0.f : 1.f / l_tot;
  uint16_t* op = p.o + ((size_t)(b * p.h + head) * p.T_q + qrow) * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + half * 4;
      float v0 = acc[db][g4 * 4 + 0] * inv, v1 = acc[db][g4 * 4 + 1] * inv;
      float v2 = acc[db][g4 * 4 + 2] * inv, v3 = acc[db][g4 * 4 + 3] * inv;
      if (empty) v0 = v1 = v2 = v3 = 0.f;
      store8(op + d, u32x2{E::pack2(v0, v1), E::pack2(v2, v3)});
    }
  }
  if (p.lse != nullptr && half == 0)
    p.lse[(size_t)(b * p.h + head) * p.T_q + qrow] = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
}

template <int DT, bool CAUSAL, bool KMASK>
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.n_grp * p.B * p.h_kv));
  hipLaunchKernelGGL((prefill_kernel<DT, CAUSAL, KMASK>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int DT>
hipError_t dispatch_prefill(const PrefillParams& p, bool causal, bool kmask, hipStream_t s) {
  if (causal) return kmask ? launch_prefill<DT, true, true>(p, s) : launch_prefill<DT, true, false>(p, s);
  return kmask ? launch_prefill<DT, false, true>(p, s) : launch_prefill<DT, false, false>(p, s);
}

}  // namespace

hipError_t prefill_fwd(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                       const uint8_t* row_mask, void* o, float* lse, int B, int h, int h_kv,
                       int T_q, int T_k, int dtype, float scale, int causal, hipStream_t stream) {
  PrefillParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.key_mask = key_mask;
  p.row_mask = row_mask;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B;
  p.h = h;
  p.h_kv = h_kv;
  p.T_q = T_q;
  p.T_k = T_k;
  p.g = h / h_kv;
  p.n_rb = p.g * ((T_q + kRows - 1) / kRows);
  p.n_grp = (p.n_rb + kWaves - 1) / kWaves;
  p.c = scale * kLog2e;
  if (B == 0 || T_q == 0 || h == 0) return hipSuccess;
  if (dtype == ATTN_DTYPE_BF16) return dispatch_prefill<ATTN_DTYPE_BF16>(p, causal != 0, key_mask != nullptr, stream);
  return dispatch_prefill<ATTN_DTYPE_F16>(p, causal != 0, key_mask != nullptr, stream);
}

}  // namespace attn
