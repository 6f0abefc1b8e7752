// Split-KV decode (stage 1) for gfx950, and the host-side split plan.
//
// "Decode attention: FlashDecoding, split-K, paged kernels": with one query
// token per sequence the query axis gives almost no parallelism, so the key
// axis is cut into contiguous slices, each slice runs the online-softmax loop
// over its own keys, and each emits an unnormalised partial state (O~, m, l)
// that a second kernel merges (opening section; section "Segment length, and
// the early exit"). All g query heads of a KV head are handled by one
// workgroup, so each K/V byte is read from HBM once (section "Where GQA
// enters"). Paged KV is addressed through the block table: key p of sequence
// b is slot p % P of page table[b][p / P] (the paged addressing after
// section "What the merge costs").
//
// Workgroup = one (sequence b, KV head, split); with up to 16 query heads
// per KV head (key mode) its 4 waves take 32-key tiles of the split
// round-robin, each with its own state, and merge the four states through
// LDS at the end.
//
// Groups of more than 16 query heads (g up to 256; 128 for MLA-style models)
// are tiled into ceil(g / 16) head blocks, as the pages' grouped-head decode
// does ("Decode attention: FlashDecoding, split-K, paged kernels", section
// "SGLang: a split count computed per sequence, on device": 16 heads per
// block, the group tiled across blocks). Then each wave of a workgroup takes
// one head block and walks every tile of the split (head mode), so the four
// waves read the same keys at the same time and each ends with a complete
// state; a group of more than 4 head blocks spreads over several workgroups.
// The library sends groups of more than 16 heads to the prefill kernel
// instead (the heads as its MFMA rows), except on a paged cache whose page
// size is not a power of two: head mode serves those.
//
// Per 32-key tile and wave (v_mfma_f32_16x16x32, the up to 16 query heads of
// the head block as the 16 columns, unused columns zero):
// K and V are read exactly once, with non-temporal loads (on the 64-sequence
// paged workload 5.69 TB/s against 5.34-5.50 with ordinary loads).
//   S^T = K Q^T: A = K rows loaded straight from global memory (lane l: key
//   l%16 of a 16-key block, d in [8*(l/16) + 32c, +8)), B = Q^T in VGPRs.
//   Accumulator: lane l holds head l%16 and keys 4*(l/16) + r of the block.
//   Row max: in-lane over 8 scores, then across the four 16-lane rows (lane
//   swaps). The reference that the weights are taken against lags the
//   running maximum by up to 2^8, so O~ is rescaled only on the few tiles
//   where a head's maximum passes it by more.
//   O~^T += V^T P^T: P^T comes from the score registers as the B operand
//   (keys 4a+r of block 0 then of block 1, a = l/16); V rows are stored as
//   they are in a per-wave LDS region, and the A operand (8 keys of one d)
//   is read with two of gfx950's transposing 8-byte LDS reads.
// Keys outside the split, past the sequence, or on a page id outside the
// pool are excluded (score -inf) and their V rows are zeroed before use, so
// poisoned (NaN) slots never reach the result.
//
// 8-bit K/V (KV8; "The Online Softmax Recurrence", section "Where it
// breaks": FP8 operands with fp32 statistics). K and V hold OCP E4M3 codes
// with one fp32 scale per tensor. The codes become MFMA operands in
// registers (K in the query's type, V in fp16, both exact); k_scale joins
// the score constant and v_scale the factor each split's O~ is written
// with. The loads of each wave's next two tiles stay in flight while a tile
// is computed (see the KV8 loop).
#include <type_traits>

#include "common.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kTile = 32;              // keys per wave tile
constexpr float kTau = 8.f;            // allowed lag of the reference max (log2 units)
// V tile in LDS, one key row per 288 bytes: consecutive rows start 8 banks
// apart, so the 4 rows x 32 bytes of a 16-lane transposing read never share
// a bank.
constexpr int kVrStr = kD + 16;
constexpr int kWaveLds = kTile * kVrStr;  // elements per wave region

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* bt;
  const int32_t* seq_lens;
  float* part_o;
  float* part_m;
  float* part_l;
  int max_pages, page_size, num_pages;
  int s_max;
  int B, h, h_kv, g;
  int n_hb;    // head blocks of 16 per KV head = ceil(g / 16)
  int chunk, max_splits;
  float c;     // scale * log2(e) (times k_scale for 8-bit K/V)
  float v_scale;   // 8-bit K/V: V's tensor scale, applied to O~ as it is written
};

// Max / sum of x over the four 16-lane rows of a wave (lanes l, l^16,
// l^32, l^48), by the lane swaps (no LDS round trip); every lane gets the
// same bits (sums add the lower row first).
__device__ __forceinline__ float max_rows16(float x) {
  float lo, hi;
  swap_rows16(x, lo, hi);
  return max_halves(fmaxf(lo, hi));
}
__device__ __forceinline__ float sum_rows16(float x) {
  float lo, hi;
  swap_rows16(x, lo, hi);
  return sum_halves(lo + hi);
}


// STREAM: K/V loads carry the non-temporal hint (each byte read once). In
// head mode the waves of a workgroup (and, beyond 4 head blocks, several
// workgroups) read the same keys, and the loads must leave them in the
// caches.
// Paged 8-bit forms: at most 168 registers, 3 workgroups per CU (they fit
// without spills). The contiguous 8-bit forms take a few more; they serve
// batches of few long sequences, where the grid fills one workgroup per CU.
template <int DT, bool PAGED, bool STREAM, bool KV8>
__global__ __launch_bounds__(256, KV8 && PAGED ? 3 : 2) void decode_split_kernel(DecodeParams p) {
  using E = Elem<DT>;
  // The PV product: on the operand type with 8-bit V it is fp16 whatever the
  // query type (E4M3 codes, at most 448 in magnitude, are exact fp16 values,
  // and P rounded to fp16 keeps 3 more bits than bf16).
  constexpr int PDT = KV8 ? ATTN_DTYPE_F16 : DT;
  using EP = Elem<PDT>;
  using KE = std::conditional_t<KV8, uint8_t, uint16_t>;   // stored K/V element
  const KE* const k_el = reinterpret_cast<const KE*>(p.k);
  const KE* const v_el = reinterpret_cast<const KE*>(p.v);
  __shared__ __attribute__((aligned(16))) uint16_t lds[kWaves * kWaveLds];

  // Consecutive workgroups (dealt round-robin to the 8 XCDs) take
  // consecutive splits of one (sequence, head), rotated by (head + sequence)
  // so that the split index does not follow the XCD: otherwise, with a
  // multiple of 8 splits, one XCD would get every sequence's split 0 and
  // another only the longest sequences' last splits.
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Head mode (more than one head block of 16): the 4 waves of a workgroup
  // take 4 head blocks of the group and each walks every tile of the split,
  // so the four read the same keys together (one fetch, three L1 hits) and
  // each ends with the complete state of its 16 heads. Otherwise (key mode)
  // the 4 waves share one head block and take the tiles round-robin.
  const bool head_mode = p.n_hb > 1;
  unsigned gx = blockIdx.x, gy = blockIdx.y, gz = blockIdx.z;
  int hb = 0;
  if (head_mode) {
    // 1-D grid: the n_hg head groups of one (split, KV head, sequence) unit
    // sit 8 apart in launch order, so they land on the same XCD close in
    // time and re-read the unit's keys from that XCD's L2.
    const unsigned n_hg = (unsigned)(p.n_hb + kWaves - 1) / kWaves;
    const unsigned L = blockIdx.x;
    hb = (int)((L >> 3) % n_hg) * kWaves + __builtin_amdgcn_readfirstlane(wave);
    const unsigned u = (L & 7u) + 8u * (L / (8u * n_hg));
    if (u >= (unsigned)(p.max_splits * p.h_kv * p.B) || hb >= p.n_hb) return;   // no barrier in head mode
    gx = u % (unsigned)p.max_splits;
    gy = (u / (unsigned)p.max_splits) % (unsigned)p.h_kv;
    gz = u / ((unsigned)p.max_splits * (unsigned)p.h_kv);
  }
  const int kvh = (int)gy;
  const int hb0 = hb * 16;               // first head of this block in the group
  const int hn = min(16, p.g - hb0);     // heads in this block
  const int b = (int)gz;
  const int split = (int)((gx + gy + gz) % (unsigned)p.max_splits);
#ifdef ATTN_DEVICE_CHECKS
  // extents of the tensors, in bytes
  const size_t q_bytes = (size_t)p.B * p.h * kD * 2;
  const size_t kv_bytes = (PAGED ? (size_t)p.num_pages * p.page_size : (size_t)p.B * p.s_max) * p.h_kv * kD * sizeof(KE);
  const size_t bt_bytes = (size_t)p.B * p.max_pages * 4;
  const size_t part_rows = (size_t)p.B * p.h * p.max_splits;
#endif
  const int s_raw = ATTN_IN_RANGE(p.seq_lens + b, 4, p.seq_lens, (size_t)p.B * 4, kSiteDecSeqLens) ? p.seq_lens[b] : 0;
  if (s_raw <= 0) return;
  const int n_split = min(p.max_splits, (s_raw + p.chunk - 1) / p.chunk);
  if (split >= n_split) return;
  const int cap = PAGED ? p.max_pages * p.page_size : p.s_max;
  const int s_len = min(s_raw, cap);
  const int k_lo = split * p.chunk;
  const int k_hi = split == p.max_splits - 1 ? s_len : min(s_len, k_lo + p.chunk);

  const int col = lane & 15;   // query head inside the group
  const int row = lane >> 4;   // 16-lane row 0..3

  // Q^T as B operands: lane holds head col and one d-chunk of 8 per step.
  u32x4 qf[4];
  {
    const bool ok = col < hn;
    const uint16_t* qh = p.q + ((size_t)b * p.h + kvh * p.g + hb0 + (ok ? col : 0)) * kD;
    // MFMA step c sums over d-chunk row + 4c (8-bit K/V: 2 row + (c & 1) +
    // 8 (c >> 1), the chunks a lane's 16-byte K loads hold); the order of
    // the d-chunks over the steps does not change the sum's terms
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int chunk = KV8 ? 2 * row + (c & 1) + 8 * (c >> 1) : row + 4 * c;
      qf[c] = ok && ATTN_IN_RANGE(qh + chunk * 8, 16, p.q, q_bytes, kSiteDecQ) ? load16(qh + chunk * 8)
                                                                               : u32x4{0, 0, 0, 0};
    }
  }

  const long kstride = PAGED ? p.h_kv : 1;   // rows between consecutive keys

  uint16_t* vt = lds + wave * kWaveLds;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{};
  float m_run = -INFINITY;
  float l_run = 0.f;   // replicated across the 4 rows after reduction
  // Sum of the weights as rounded for the PV product. The split's O~ is
  // written scaled by l / l~, so that with part_l = l (fp32 weights, for the
  // LSE) the merge divides the rounded-weight products by their own sum.
  float lr_run = 0.f;

  const int n_tiles = (k_hi - k_lo + kTile - 1) / kTile;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int t0 = head_mode ? 0 : wave_u;
  const int dt = head_mode ? 1 : kWaves;
  // Page rows and validity of the two 16-key blocks of tile t.
  auto tile_rows = [&](int kt, long (&rbase)[2], bool (&bok)[2]) {
    // Each 16-key block lies inside one page (pages hold a multiple of 16
    // keys and blocks start at multiples of 16): resolve its row once.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key0 = kt + kb * 16;
      bok[kb] = key0 < k_hi;
      if (PAGED) {
        const int32_t* pe = p.bt + (size_t)b * p.max_pages + key0 / p.page_size;
        int page = bok[kb] && ATTN_IN_RANGE(pe, 4, p.bt, bt_bytes, kSiteDecTable) ? *pe : 0;
        page = __builtin_amdgcn_readfirstlane(page);
        bok[kb] = bok[kb] && page >= 0 && page < p.num_pages;
        rbase[kb] = ((long)(bok[kb] ? page : 0) * p.page_size + key0 % p.page_size) * p.h_kv + kvh;
      } else {
        rbase[kb] = ((long)b * p.h_kv + kvh) * p.s_max + key0;
      }
    }
  };
  // QK, softmax, V^T staging and PV of one tile, from 16-bit operands.
  // K fragments come from kfrag(kb, c), word e of V row i from vword(i, e); after_stage()
  // runs once the tile's K and V registers are consumed (after the V^T
  // stores), so the 8-bit path can reuse them for the next loads.
  auto tile_compute = [&](int kt, const bool (&bok_in)[2], auto&& kfrag, auto&& vword, auto&& after_stage) {
    const bool bok[2] = {bok_in[0], bok_in[1]};
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int c = 0; c < 4; ++c) s[kb] = E::mfma16(kfrag(kb, c), qf[c], s[kb]);
    }
    // Exclude keys outside [k_lo, k_hi) or on an invalid page: register r of
    // block kb holds key kt + 16kb + 4row + r. Only the last tile of a split
    // and tiles on an invalid page need it (the test is wave-uniform).
    if (!(bok[0] && bok[1] && kt + kTile <= k_hi)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = bok[kb] && kt + kb * 16 + row * 4 + r < k_hi;
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
      }
    }

    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max_rows16(mx);
    // Lagging reference ("The Online Softmax Recurrence", section "The
    // recurrence": any reference gives the same state once merged): m_run
    // moves only when a head's largest logit exceeds it by more than kTau,
    // so every weight stays below 2^kTau and O~ is rescaled on few tiles.
    const float mr = mx * p.c;
    const bool move = mr > m_run + kTau;
    const float alpha = move ? fast_exp2(m_run - mr) : 1.f;   // m_run = -inf: 0
    m_run = move ? mr : m_run;
    const float base = m_run == -INFINITY ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(__builtin_fmaf(s[kb][r], p.c, -base));
        s[kb][r] = e;
        rs += e;
      }
    }
    l_run = l_run * alpha + sum_rows16(rs);
    if (__ballot(move)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
    }

    // Stage V: lane (col = d-chunk, row = key group) stores its 8 key rows
    // (keys 4row+i and 16+4row+i) as they are, 16 bytes each.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = (i < 4 ? 0 : 16) + row * 4 + (i & 3);
      store16(&vt[key * kVrStr + col * 8], u32x4{vword(i, 0), vword(i, 1), vword(i, 2), vword(i, 3)});
    }
    after_stage();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const u32x4 pf = u32x4{EP::pack2(s[0][0], s[0][1]), EP::pack2(s[0][2], s[0][3]),
                           EP::pack2(s[1][0], s[1][1]), EP::pack2(s[1][2], s[1][3])};
    lr_run = lr_run * alpha +
             sum_rows16(EP::add_pair(pf[3], EP::add_pair(pf[2], EP::add_pair(pf[1], EP::add_pair(pf[0], 0.f)))));
    // A operand V^T (d = 16db + col, keys 4row..4row+3 and 16+4row..+3, the
    // key order of P^T) by transposing reads: lane (col, row) addresses key
    // row 4row + col/4 (and 16 + that), d 16db + 4(col % 4), and receives
    // element col % 4 of lanes 4k + col/4, i.e. d = 16db + col of keys
    // 4row + k.
    const uint16_t* vlo = vt + (row * 4 + (col >> 2)) * kVrStr + 4 * (col & 3);
    const uint16_t* vhi = vlo + 16 * kVrStr;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2 lo = lds_read_tr16(vlo + 16 * db);
      const u32x2 hi = lds_read_tr16(vhi + 16 * db);
      acc[db] = EP::mfma16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, acc[db]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if constexpr (!KV8) {
    for (int t = t0; t < n_tiles; t += dt) {
      const int kt = k_lo + t * kTile;
      long rbase[2];
      bool bok[2];
      tile_rows(kt, rbase, bok);
      // K: lane loads key 16kb + col, d-chunks 8*row + 32c.
      u32x4 kf[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool ok = bok[kb] && kt + kb * 16 + col < k_hi;
        const KE* kp = k_el + (rbase[kb] + (ok ? col : 0) * kstride) * kD + row * 8;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          kf[kb][c] = ok && ATTN_IN_RANGE(kp + c * 32, 16, p.k, kv_bytes, kSiteDecK16)
                          ? (STREAM ? load16_nt(kp + c * 32) : load16(kp + c * 32))
                          : u32x4{0, 0, 0, 0};
      }
      // V: lane (d-chunk col, key group row) loads keys 4*row+i and 16+4*row+i.
      u32x4 vf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kb = i >> 2;
        const int ko = row * 4 + (i & 3);
        const bool ok = bok[kb] && kt + kb * 16 + ko < k_hi;
        const KE* vp = v_el + (rbase[kb] + ko * kstride) * kD + col * 8;
        vf[i] = ok && ATTN_IN_RANGE(vp, 16, p.v, kv_bytes, kSiteDecV16) ? (STREAM ? load16_nt(vp) : load16(vp))
                                                                        : u32x4{0, 0, 0, 0};
      }

      tile_compute(
          kt, bok, [&](int kb, int c) { return kf[kb][c]; }, [&](int i, int e) { return vf[i][e]; }, [] {});
    }
  } else {
    // 8-bit K/V, software-pipelined: each wave keeps the loads of its next
    // two tiles in flight. A tile's registers are refilled with the loads of
    // the tile two steps on as soon as its K and V have been converted and
    // staged, before its PV product, so the loads run under the compute.
    // Every load is an unconditional buffer load: a 16-key block gets a
    // buffer resource whose range ends after its last key in bounds (none
    // for a block past the split or on a page outside the pool), so keys out
    // of range read as zeros with no branch, and the load counter waits can
    // name the exact tile they need. The page ids of a tile's two blocks
    // (lanes 0 and 1 of one vector load) are read one step ahead, in the
    // same in-order stream as the tile loads.
    // K: lane (key col, row) loads 16 codes, bytes [16 (row + 4 hh), +16) of
    // its key; MFMA step c takes d-chunk 2 row + (c & 1) + 8 (c >> 1), as Q.
    // V: lane (d-chunk col, key group row) loads 8 codes of keys 4 row + i
    // and 16 + 4 row + i.
    struct Raw {
      u32x4 k[2][2];
      u32x2 v[8];
      bool bok[2];
    };
    constexpr int kAux = STREAM ? 2 : 0;   // buffer-load cache policy: nt
    const bool bt_ok = !PAGED || ATTN_IN_RANGE(p.bt + (size_t)b * p.max_pages, (size_t)p.max_pages * 4, p.bt, bt_bytes,
                                               kSiteDecTable8);
    const __amdgpu_buffer_rsrc_t r_bt =
        make_rsrc(PAGED ? p.bt + (size_t)b * p.max_pages : p.bt, PAGED && bt_ok ? (uint32_t)p.max_pages * 4u : 0u);
    // Paged: a cursor per use walks one slot's tiles (every (2 dt)-th tile
    // of the wave) as (table index, key offset in the page) of the tile's
    // first key, advanced by adds instead of a division per tile. Blocks
    // start at multiples of 16 keys and pages hold multiples of 16, so a
    // tile's second block is 16 keys on, in the same page or at the start of
    // the next. Entries past the table read as zero through r_bt's range;
    // their keys lie past the sequence and are excluded anyway.
    struct Cursor {
      int idx, off;
    };
    const int ps = PAGED ? p.page_size : 16;
    const int slot_keys = 2 * dt * kTile;
    const int adv_pages = PAGED ? slot_keys / ps : 0, adv_keys = PAGED ? slot_keys % ps : 0;
    auto cursor_at = [&](int t) {
      const int key0 = k_lo + t * kTile;
      return Cursor{PAGED ? key0 / ps : 0, PAGED ? key0 % ps : 0};
    };
    auto advance = [&](Cursor& c) {
      c.idx += adv_pages;
      c.off += adv_keys;
      if (c.off >= ps) {
        c.off -= ps;
        ++c.idx;
      }
    };
    // page ids of the tile at cursor c: block 0 on lane 0, block 1 on lane 1
    auto page_load = [&](Cursor& c) -> int {
      if constexpr (!PAGED) return 0;
      const int i1 = c.idx + (c.off + 16 >= ps ? 1 : 0);
      const int pg = (int)__builtin_amdgcn_raw_buffer_load_b32(r_bt, ((lane & 1) ? i1 : c.idx) * 4, 0, 0);
      advance(c);
      return pg;
    };
    // per-lane byte offsets inside a block (all in the vector offset, which
    // the range check covers)
    const int row_bytes = (int)kstride * kD;
    const int k_off = col * row_bytes + row * 16;
    const int v_off = row * 4 * row_bytes + col * 8;
    auto issue = [&](int t, int pg, Cursor& c, Raw& r) {
      const int kt = k_lo + t * kTile;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key0 = kt + kb * 16;
        bool ok = key0 < k_hi;
        long rb;
        if (PAGED) {
          const int page = __builtin_amdgcn_readlane(pg, kb);
          ok = ok && page >= 0 && page < p.num_pages;
          const int off = kb == 0 ? c.off : (c.off + 16 >= ps ? c.off + 16 - ps : c.off + 16);
          rb = ((long)(ok ? page : 0) * ps + off) * p.h_kv + kvh;
        } else {
          rb = ((long)b * p.h_kv + kvh) * p.s_max + key0;
        }
        const int nv = ok ? min(16, k_hi - key0) : 0;
        r.bok[kb] = ok;
        uint32_t bytes = nv > 0 ? (uint32_t)(((long)(nv - 1) * kstride + 1) * kD) : 0u;
        if (bytes != 0 && !(ATTN_IN_RANGE(k_el + rb * kD, bytes, p.k, kv_bytes, kSiteDecK8) &&
                            ATTN_IN_RANGE(v_el + rb * kD, bytes, p.v, kv_bytes, kSiteDecV8)))
          bytes = 0u;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(k_el + rb * kD, bytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(v_el + rb * kD, bytes);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          r.k[kb][hh] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off + 64 * hh, 0, kAux));
#pragma unroll
        for (int i = 0; i < 4; ++i)
          r.v[kb * 4 + i] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(vr, v_off + i * row_bytes, 0, kAux));
      }
      if (PAGED) advance(c);
    };
    auto compute8 = [&](int t, Raw& r, auto&& refill) {
      tile_compute(
          k_lo + t * kTile, r.bok,
          [&](int kb, int c) {
            const u32x4 w = r.k[kb][c >> 1];
            return (c & 1) ? cvt8<DT>(u32x2{w[2], w[3]}) : cvt8<DT>(u32x2{w[0], w[1]});
          },
          [&](int i, int e) { return cvt8w<PDT>(r.v[i][e >> 1], e & 1); }, refill);
    };
    Raw ra, rb;
    // load cursors (la, lb) run one slot tile ahead of the issue cursors
    Cursor la = cursor_at(t0), lb = cursor_at(t0 + dt), ia = la, ib = lb;
    int pga = page_load(la), pgb = page_load(lb);
    __builtin_amdgcn_sched_barrier(0);
    issue(t0, pga, ia, ra);
    __builtin_amdgcn_sched_barrier(0);
    pga = page_load(la);
    __builtin_amdgcn_sched_barrier(0);
    issue(t0 + dt, pgb, ib, rb);
    __builtin_amdgcn_sched_barrier(0);
    pgb = page_load(lb);
    __builtin_amdgcn_sched_barrier(0);
    // Whole pairs in the loop, so that its back edge is reached only after
    // both refills were issued (the load-counter waits at the loop head then
    // count exactly the loads issued since); an odd last tile after it.
    int t = t0;
    for (; t + dt < n_tiles; t += 2 * dt) {
      compute8(t, ra, [&] {
        __builtin_amdgcn_sched_barrier(0);
        issue(t + 2 * dt, pga, ia, ra);
        __builtin_amdgcn_sched_barrier(0);
        pga = page_load(la);
        __builtin_amdgcn_sched_barrier(0);
      });
      compute8(t + dt, rb, [&] {
        __builtin_amdgcn_sched_barrier(0);
        issue(t + 3 * dt, pgb, ib, rb);
        __builtin_amdgcn_sched_barrier(0);
        pgb = page_load(lb);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    if (t < n_tiles) compute8(t, ra, [] {});
  }

  if (head_mode) {
    // This wave's state is complete: write its 16 heads' partials.
    // acc[db] lane (col, row) reg r: head col, d = 16db + 4row + r
    if (col < hn) {
      const size_t hs = (size_t)b * p.h + kvh * p.g + hb0 + col;
      float* po = p.part_o + (hs * p.max_splits + split) * kD;
      float f = lr_run > 0.f ? l_run / lr_run : 1.f;
      if (KV8) f *= p.v_scale;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        if (ATTN_IN_RANGE(&po[db * 16 + row * 4], 16, p.part_o, part_rows * kD * 4, kSiteDecPartO))
          *reinterpret_cast<f32x4*>(&po[db * 16 + row * 4]) = acc[db] * f;
      if (row == 0 && ATTN_IN_RANGE(p.part_m + hs * p.max_splits + split, 4, p.part_m, part_rows * 4, kSiteDecPartML) &&
          ATTN_IN_RANGE(p.part_l + hs * p.max_splits + split, 4, p.part_l, part_rows * 4, kSiteDecPartML)) {
        p.part_m[hs * p.max_splits + split] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
        p.part_l[hs * p.max_splits + split] = l_run;
      }
    }
    return;
  }

  // Merge the 4 wave states through LDS. Each wave writes its state into its
  // own V region, which no other wave uses, once its own tiles are done: [16
  // heads][128 d] then [16][3] (m, l, l~). One barrier, before the reads.
  static_assert((16 * kD + 16 * 3) * 4 <= kWaveLds * 2, "a wave's state fits its V region");
  auto red_of = [&](int w) { return reinterpret_cast<float*>(lds + w * kWaveLds); };
  {
    float* r = red_of(wave);
    // acc[db] lane (col, row) reg r: head col, d = 16db + 4row + r
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(&r[col * kD + db * 16 + row * 4]) = acc[db];
    if (row == 0) {
      r[16 * kD + col * 3 + 0] = m_run;
      r[16 * kD + col * 3 + 1] = l_run;
      r[16 * kD + col * 3 + 2] = lr_run;
    }
  }
  __syncthreads();

  // 256 threads: head j = tid / 32 (+8 per pass), 4 d-values each.
  for (int j = tid >> 5; j < hn; j += 8) {
    const int d = (tid & 31) * 4;
    float mw[kWaves], m_all = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = red_of(w)[16 * kD + j * 3];
      m_all = fmaxf(m_all, mw[w]);
    }
    f32x4 o = f32x4{};
    float l_all = 0.f, lr_all = 0.f;
    if (m_all != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = fast_exp2(mw[w] - m_all);   // empty wave: 2^-inf = 0
        l_all += wt * red_of(w)[16 * kD + j * 3 + 1];
        lr_all += wt * red_of(w)[16 * kD + j * 3 + 2];
        o += wt * *reinterpret_cast<const f32x4*>(&red_of(w)[j * kD + d]);
      }
    }
    float f = lr_all > 0.f ? l_all / lr_all : 1.f;
    if (KV8) f *= p.v_scale;
    const size_t hs = (size_t)b * p.h + kvh * p.g + hb0 + j;
    if (ATTN_IN_RANGE(&p.part_o[(hs * p.max_splits + split) * kD + d], 16, p.part_o, part_rows * kD * 4,
                      kSiteDecPartO))
      *reinterpret_cast<f32x4*>(&p.part_o[(hs * p.max_splits + split) * kD + d]) = o * f;
    if ((tid & 31) == 0 &&
        ATTN_IN_RANGE(p.part_m + hs * p.max_splits + split, 4, p.part_m, part_rows * 4, kSiteDecPartML) &&
        ATTN_IN_RANGE(p.part_l + hs * p.max_splits + split, 4, p.part_l, part_rows * 4, kSiteDecPartML)) {
      p.part_m[hs * p.max_splits + split] = m_all == -INFINITY ? -INFINITY : m_all * kLn2;
      p.part_l[hs * p.max_splits + split] = l_all;
    }
  }
}

template <int DT, bool KV8>
hipError_t dispatch_decode(const DecodeParams& p, bool paged, hipStream_t stream) {
  const long units = (long)p.max_splits * p.h_kv * p.B;
  const long n_hg = (p.n_hb + kWaves - 1) / kWaves;
  const dim3 grid = p.n_hb == 1 ? dim3((unsigned)p.max_splits, (unsigned)p.h_kv, (unsigned)p.B)
                                : dim3((unsigned)(((units + 7) / 8) * 8 * n_hg));
  const bool stream_kv = p.n_hb == 1;
  if (paged) {
    if (stream_kv) hipLaunchKernelGGL((decode_split_kernel<DT, true, true, KV8>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_split_kernel<DT, true, false, KV8>), grid, dim3(256), 0, stream, p);
  } else {
    if (stream_kv) hipLaunchKernelGGL((decode_split_kernel<DT, false, true, KV8>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_split_kernel<DT, false, false, KV8>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

namespace {
DecodeParams decode_params(const void* q, const void* k, const void* v, const int32_t* block_table,
                           int max_pages, int page_size, int num_pages, const int32_t* seq_lens, int s_max,
                           int B, int h, int h_kv, int chunk_keys, int max_splits, float scale, float* part_o,
                           float* part_m, float* part_l) {
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.bt = block_table;
  p.seq_lens = seq_lens;
  p.part_o = part_o;
  p.part_m = part_m;
  p.part_l = part_l;
  p.max_pages = max_pages;
  p.page_size = page_size;
  p.num_pages = num_pages;
  p.s_max = s_max;
  p.B = B;
  p.h = h;
  p.h_kv = h_kv;
  p.g = h / h_kv;
  p.n_hb = (p.g + 15) / 16;
  p.chunk = chunk_keys;
  p.max_splits = max_splits;
  p.c = scale * kLog2e;
  p.v_scale = 1.f;
  return p;
}
}  // namespace

ATTN_DEFINE_CHECK_READER(decode)

hipError_t decode_split(const void* q, const void* k, const void* v, const int32_t* block_table,
                        int max_pages, int page_size, int num_pages, const int32_t* seq_lens,
                        int s_max, int B, int h, int h_kv, int chunk_keys, int max_splits,
                        int dtype, float scale, float* part_o, float* part_m, float* part_l,
                        hipStream_t stream) {
  const DecodeParams p = decode_params(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B,
                                       h, h_kv, chunk_keys, max_splits, scale, part_o, part_m, part_l);
  if (B == 0 || h == 0) return hipSuccess;
  if (dtype == ATTN_DTYPE_BF16) return dispatch_decode<ATTN_DTYPE_BF16, false>(p, block_table != nullptr, stream);
  return dispatch_decode<ATTN_DTYPE_F16, false>(p, block_table != nullptr, stream);
}

// 8-bit E4M3 K/V with per-tensor scales: k_scale joins the logit scale (the
// scores are (q . k_code) * k_scale * scale), v_scale multiplies each
// split's O~ (l and m do not involve V). Every group size runs on this
// file's kernel (head blocks of 16 beyond 16 query heads per KV head).
hipError_t decode_split_fp8kv(const void* q, const void* k, const void* v, const int32_t* block_table,
                             int max_pages, int page_size, int num_pages, const int32_t* seq_lens, int s_max,
                             int B, int h, int h_kv, int chunk_keys, int max_splits, int dtype, float scale,
                             float k_scale, float v_scale, float* part_o, float* part_m, float* part_l,
                             hipStream_t stream) {
  DecodeParams p = decode_params(q, k, v, block_table, max_pages, page_size, num_pages, seq_lens, s_max, B, h,
                                 h_kv, chunk_keys, max_splits, scale, part_o, part_m, part_l);
  p.c = scale * k_scale * kLog2e;
  p.v_scale = v_scale;
  if (B == 0 || h == 0) return hipSuccess;
  if (dtype == ATTN_DTYPE_BF16) return dispatch_decode<ATTN_DTYPE_BF16, true>(p, block_table != nullptr, stream);
  return dispatch_decode<ATTN_DTYPE_F16, true>(p, block_table != nullptr, stream);
}

// Split plan. The unsplit grid has B * h_kv workgroups; the split count that
// first fills the machine is ceil(num_cus / (B * h_kv)) ("Decode attention:
// FlashDecoding, split-K, paged kernels", section "The grid"). Here the key
// slice length is chosen instead, so ragged batches are balanced too: aim at
// wgs_per_cu workgroups per CU of total work. For this file's kernel, 12
// (several per CU keep enough loads in flight and even out ragged lengths;
// fewer, longer slices spend less on each workgroup's start and final merge
// -- on the 64-sequence Llama-3-8B shape 1280-key slices read 5.5 TB/s where
// 960-key slices read 5.2); for the prefill kernel's row form, which runs one
// workgroup per CU, 1. Never below 128 keys per slice unless that is needed
// to reach one workgroup per CU, never below 64.
// units_per_split: workgroups one split launches (one per KV head).
int decode_plan(int B, const int32_t* seq_lens, int units_per_split, int wgs_per_cu, int num_cus, int32_t* chunk_keys,
                int32_t* max_splits) {
  long total = 0;
  int s_max = 0;
  for (int b = 0; b < B; ++b) {
    total += seq_lens[b];
    s_max = seq_lens[b] > s_max ? seq_lens[b] : s_max;
  }
  auto units = [&](long chunk) {
    long u = 0;
    for (int b = 0; b < B; ++b) u += (seq_lens[b] + chunk - 1) / chunk;
    return u * units_per_split;
  };
  const long target = (long)wgs_per_cu * num_cus;
  long chunk = (total * units_per_split + target - 1) / target;
  chunk = ((chunk + 63) / 64) * 64;
  if (chunk < 128) chunk = 128;
  while (chunk > 64 && units(chunk) < num_cus) chunk -= 64;
  if (chunk < 64) chunk = 64;
  *chunk_keys = (int32_t)chunk;
  long ms = (s_max + chunk - 1) / chunk;
  *max_splits = (int32_t)(ms < 1 ? 1 : ms);
  return 0;
}

}  // namespace attn
