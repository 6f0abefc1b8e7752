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
//   K and V tiles are staged into LDS in their natural row-major layout with
//   range-checked buffer loads (rows past T_k read as zeros), double
//   buffered, one barrier per tile.
//   S^T = K Q^T on v_mfma_f32_32x32x16 (A = K rows from LDS, B = the wave's
//   Q rows held in VGPRs for the whole kernel). In the accumulator layout
//   lane l holds query row l%32 and, for register r of 32-key block kb, key
//   kb*32 + 8*(r/4) + 4*(l/32) + r%4.
//   O~^T += V^T P^T on the same MFMA: P^T is the B operand straight from the
//   score registers (rounded to the operand dtype; the 8 keys of lane group
//   h in 16-key chunk cc are 16cc + 4h + {0..3} and 16cc + 8 + 4h + {0..3});
//   the V^T A operand is two transposing LDS reads of 4 consecutive keys x 1
//   column each from the natural V tile.
//
// Online softmax in base 2, c = scale * log2(e): p = 2^(c*s - m) where m is
// the row's reference maximum. The reference moves only when a score exceeds
// it by more than kTau (then m <- the row's new maximum and l, O~ are
// multiplied by alpha = 2^(m_old - m_new)); otherwise p <= 2^kTau and no
// rescale is done. This is the recurrence of the pages with a reference that
// is allowed to lag the running maximum: every term stays relative to the
// same m in l and O~, so the result is unchanged in exact arithmetic, and
// p <= 2^8 fits the fp32 state and the fp16/bf16 operands. While a row has
// seen no visible key its reference stays -inf and the subtracted value is
// 0, so -inf - (-inf) is never formed ("Merge normalized attention without
// averaging tile outputs", paragraph on fully masked tiles).
//   Masking (causal, key range, key mask) is applied only in tiles that need
//   it; tiles with no visible key for a wave are skipped.
//
// Two running sums per row: l, the fp32 sum of the weights p (for the LSE),
// and l~, the sum of the weights as rounded to the operand dtype for the PV
// product. O~ accumulates the rounded weights, so it is divided by l~: the
// output is then an exact convex combination of the value rows with weights
// p~ / l~, whatever the magnitude of the dominant weight (up to 2^kTau here).
//
// Epilogue: O = O~/l~ rounded to the output dtype, LSE = (m + log2 l) ln 2.
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
// LDS row strides. K rows are read 16 B per lane along a row; 272 B rows put
// the 32 rows of a fragment read on distinct bank groups. V rows are read by
// the transposing 8 B reads, which fetch 4 rows x 64 B per group of 16 lanes;
// with the 64 banks of gfx950's LDS, a 320 B stride (80 banks, 16 mod 64)
// places those 4 row segments on disjoint banks, where 288 B rows collided
// (measured: bank conflicts 3.4e7 -> 0 per launch at T = 8192).
constexpr int kKStr = kD + 8;       // 272 B
constexpr int kVStr = kD + 32;      // 320 B
constexpr int kKElems = kBc * kKStr;
constexpr int kVElems = kBc * kVStr;
constexpr float kTau = 8.f;         // allowed lag of the reference max (log2 units)

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

template <int DT, bool CAUSAL, bool KMASK>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  using E = Elem<DT>;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKElems];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kVElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
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
  // [16c + 8*half, 16c + 8*half + 8). Rows past T_q read as zeros.
  u32x4 qf[8];
  {
    const uint16_t* qbase = p.q + (size_t)(b * p.h + (wave_valid ? head : 0)) * p.T_q * kD;
    const auto rq = make_rsrc(qbase, wave_valid ? (uint32_t)p.T_q * kD * 2 : 0u);
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = buffer_load16(rq, (uint32_t)((qrow * kD + c * 16 + half * 8) * 2));
  }

  const size_t kv_base = (size_t)bk * p.T_k * kD;
  const auto rk = make_rsrc(p.k + kv_base, (uint32_t)p.T_k * kD * 2);
  const auto rv = make_rsrc(p.v + kv_base, (uint32_t)p.T_k * kD * 2);

  // Staging: 1024 16-byte chunks per tile for K and for V; chunk = tid +
  // 256 i holds key chunk / 16, d-chunk chunk % 16.
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t byte = (uint32_t)(((kt + ((tid + 256 * i) >> 4)) * kD + (tid & 15) * 8) * 2);
      kreg[i] = buffer_load16(rk, byte);
      vreg[i] = buffer_load16(rv, byte);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = (tid + 256 * i) >> 4;
      store16(&lds_k[buf][key * kKStr + (tid & 15) * 8], kreg[i]);
      store16(&lds_v[buf][key * kVStr + (tid & 15) * 8], vreg[i]);
    }
  };

  // Per-lane offsets of the transposing V reads: lane j of a 16-lane group
  // addresses key 4*half + j/4 (+8 for the upper 4 keys) and column
  // 16*((lane>>4)&1) + 4*(j%4) of each 32-column block.
  const int v_lane_off = (4 * half + ((lane & 15) >> 2)) * kVStr + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float m_ref = -INFINITY;   // reference maximum, base-2 scaled units
  float l_run = 0.f;         // this lane's share of the running sum of p
  float lr_run = 0.f;        // ... and of the rounded weights p~

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
      // QK: the 8 K fragments of a 32-key block are read before its MFMAs.
      // MFMA bursts run at raised wave priority so the other wave on the
      // SIMD fills the gaps with its softmax work instead of delaying them.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* kr = ks + (kb * 32 + col) * kKStr + half * 8;
        u32x4 kf[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) kf[c] = load16(kr + c * 16);
        s[kb] = f32x16{};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c < 8; ++c) s[kb] = E::mfma32(kf[c], qf[c], s[kb]);
        __builtin_amdgcn_s_setprio(0);
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

      // One re-reference check for the whole tile, so that the rest of the
      // tile is a single straight-line block in which the exponentials of
      // block 1 can be scheduled between the PV MFMAs of block 0.
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
      if (__ballot(mx * p.c > m_ref + kTau)) {
        const float m_new = fmaxf(m_ref, max_halves(mx) * p.c);
        if (m_new != -INFINITY) {
          const float alpha = fast_exp2(m_ref - m_new);   // m_ref = -inf -> 0
          l_run *= alpha;
          lr_run *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] *= alpha;
          m_ref = m_new;
        }
      }
      const float base = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(__builtin_fmaf(s[kb][r], p.c, -base));
          s[kb][r] = e;
          rs += e;
        }
        l_run += rs;
        // P^T for the two 16-key chunks of this block, then their PV MFMAs.
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int cc = kb * 2 + h2;
          const int r0 = h2 * 8;
          const u32x4 pf = u32x4{E::pack2(s[kb][r0 + 0], s[kb][r0 + 1]), E::pack2(s[kb][r0 + 2], s[kb][r0 + 3]),
                                 E::pack2(s[kb][r0 + 4], s[kb][r0 + 5]), E::pack2(s[kb][r0 + 6], s[kb][r0 + 7])};
          lr_run = E::add_pair(pf[3], E::add_pair(pf[2], E::add_pair(pf[1], E::add_pair(pf[0], lr_run))));
          const uint16_t* vr = vs + cc * 16 * kVStr + v_lane_off;
          u32x4 va[4];
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const u32x2 lo = lds_read_tr16(vr + db * 32);
            const u32x2 hi = lds_read_tr16(vr + 8 * kVStr + db * 32);
            va[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int db = 0; db < 4; ++db) acc[db] = E::mfma32(va[db], pf, acc[db]);
          __builtin_amdgcn_s_setprio(0);
        }
      }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_valid || qrow >= p.T_q) return;
  const float l_tot = sum_halves(l_run);
  const float lr_tot = sum_halves(lr_run);
  bool empty = l_tot == 0.f;
  if (p.row_mask != nullptr) empty = empty || p.row_mask[(size_t)b * p.T_q + qrow] == 0;
  const float inv = empty ? 0.f : 1.f / lr_tot;
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
    p.lse[(size_t)(b * p.h + head) * p.T_q + qrow] = empty ? -INFINITY : (m_ref + fast_log2(l_tot)) * kLn2;
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
