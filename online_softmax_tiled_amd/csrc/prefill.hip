// Prefill attention for gfx950: one pass over key tiles with the online
// softmax state (m, l, O~) held in registers; the score tile lives only in
// VGPRs ("Naive attention and the online softmax", sections (3) "The online
// recurrence" and "Extending the recurrence to the output").
//
// Work decomposition
//   A workgroup is 8 waves, two per SIMD, one workgroup per CU. Each wave
//   owns one block of 32 query rows of one query
//   head; the 8 blocks of a workgroup belong to query heads that share one KV
//   head (row blocks are numbered query-block-major, head-minor inside a GQA
//   group), so every K/V tile staged in LDS feeds all 8 waves. Workgroups are
//   numbered with (batch, kv head) fastest so that consecutive workgroups --
//   which the hardware deals round-robin to the 8 XCDs -- put each KV head's
//   workgroups on one XCD and its L2; the longest causal row blocks are
//   numbered first.
//
// Products, per 64-key tile and wave
//   S^T = K Q^T on v_mfma_f32_32x32x16 (A = K rows from LDS, B = the wave's
//   Q rows held in VGPRs for the whole kernel). In the accumulator layout
//   lane l holds query row l%32 and, for register r of 32-key block kb, key
//   kb*32 + 8*(r/4) + 4*(l/32) + r%4.
//   O~^T += V^T P^T on the same MFMA: P^T is the B operand straight from the
//   score registers (rounded to fp16, see below; the 8 keys of lane group
//   h in 16-key chunk cc are 16cc + 4h + {0..3} and 16cc + 8 + 4h + {0..3});
//   the V^T A operand is two transposing LDS reads of 4 consecutive keys x 1
//   column each from the natural V tile.
//
// Software pipeline
//   Iteration j issues the MFMAs of PV(j-1) and QK(j+1) and, between them,
//   the softmax of tile j, all in one straight-line block: the 32 MFMAs run
//   on the matrix core while the exponentials, sums and packing of the other
//   tile go through the VALU. The block is cut into 8 slices of 4 MFMAs, each
//   with its share of the softmax work and the LDS operand reads of the next
//   slice. Tiles stream through LDS with range-checked buffer loads (keys
//   past T_k read as zeros): K of tile t sits in slot t % 2 (read in
//   iteration t - 1), V of tile t in slot t % 3 (read in iteration t + 1);
//   K(j+2) and V(j+1) are loaded during iteration j and stored before its
//   barrier. Tiles past a wave's last visible key are fully masked, so the
//   pipeline's fill and drain iterations add exact zeros.
//
// Online softmax in base 2, c = scale * log2(e): p = 2^(c*s - m) where m is
// the row's reference maximum. The reference moves only when a score exceeds
// it by more than kTau (then m <- the row's new maximum and l, O~ are
// multiplied by alpha = 2^(m_old - m_new)); otherwise p <= 2^kTau and no
// rescale is done. This is the recurrence of the pages with a reference that
// is allowed to lag the running maximum: every term stays relative to the
// same m in l and O~, so the result is unchanged in exact arithmetic, and
// p <= 2^8 fits the fp32 state and the fp16/bf16 operands. The move is
// decided per row without branches; the rescale of O~, which must wait for
// PV(j-1), is applied at the start of the next iteration (rarely taken). While
// a row has seen no visible key its reference stays -inf and the subtracted
// value is 0, so -inf - (-inf) is never formed ("Merge normalized attention
// without averaging tile outputs", paragraph on fully masked tiles).
//
// Paged, variable-length form (PAGED)
//   The same kernel serves prefill against a paged KV cache: Q and O are
//   token-major with per-sequence offsets, T_q and T_k are read per sequence
//   on the device (bottom-right causal alignment), and K/V tiles are staged
//   through the block table, with each row's page id fetched one iteration
//   ahead. Keys on a page id outside the pool are masked through the same
//   per-tile key bits as the key mask. The host may pass a launch order of
//   the sequences (longest context first).
//
// Decode form (DEC)
//   Split-KV decode of large GQA groups: the rows are the group's query heads
//   (one token each, 32 per wave), one workgroup per (sequence, KV head,
//   split), and the epilogue writes the split's partial state for the merge.
//   With at most 128 heads (kStagers), waves 4-7 hold no rows and stage
//   every K/V tile two iterations ahead, so a CU keeps two tile pairs of
//   loads in flight while waves 0-3 compute. With 8-bit K/V (kKV8) the
//   staging waves read E4M3 codes and convert them as they store the tiles,
//   so the compute waves run the 16-bit form unchanged; k_scale is folded
//   into the score multiplier and v_scale into the epilogue's O~ factor.
//
// Paged pools under 4 GB (kPool32, paged and decode forms): K/V rows are
// addressed with range-checked 32-bit buffer offsets over the whole pool; a
// row past the keys or on a page outside the pool gets an offset past the
// range and reads zeros, with no branch and no select.
//
// Operand type of the PV product: fp16, for both input types. P is rounded
// to fp16 (11 significant bits against bf16's 8) and bf16 V is converted to
// fp16 when it is staged into LDS; every bf16 value of magnitude below 65536
// converts exactly (smaller than 2^-14 with an absolute error below 2^-24).
// With bf16 weights the error of the convex combination reaches about
// 2^-9 * sum_j w_j |v_j - O|, which with the output's own rounding (half a
// bf16 step, 2^-8 for |O| in [2, 4)) can pass 1e-2; fp16 weights cut that
// term by 8. A workgroup that stages a V value fp16 cannot hold (a bf16
// magnitude of 65536 or more) runs its pass again with bf16 operands.
//
// Two running sums per row: l, the fp32 sum of the weights p (for the LSE),
// and l~, the sum of the weights as rounded for the PV product. O~
// accumulates the rounded weights, so it is divided by l~: the output is then
// an exact convex combination of the value rows with weights p~ / l~,
// whatever the magnitude of the dominant weight (up to 2^kTau here).
//
// Epilogue: O = O~/l~ rounded to the output dtype, LSE = (m + log2 l) ln 2.
// l = 0 (no visible key) or a zero row-mask entry gives +0.0 output and
// LSE = -inf ("Merge normalized attention without averaging tile outputs",
// last paragraph).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
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
constexpr int kMaxOrder = 512;      // sequences a paged launch can reorder
constexpr int kMaxListTiles = 4096; // key-masked prefill: longest list of visible tiles

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
  int n_grp;    // workgroups per (batch, kv head) = ceil(n_rb / kWaves)
  float c;      // scale * log2(e) (times k_scale for 8-bit K/V)
  // Paged, variable-length form (PAGED): Q and O token-major [total_q, h, d]
  // with sequence b at rows cu_q[b] .. cu_q[b+1]; LSE [total_q, h]; K/V in
  // pools [num_pages, page_size, h_kv, d] addressed through the block table;
  // T_q, T_k, n_rb, n_grp above are then upper bounds over the batch and the
  // per-sequence values are read on the device.
  const int32_t* cu_q;
  const int32_t* seq_k;
  const int32_t* bt;
  int max_pages, num_pages, page_shift;   // page_size = 1 << page_shift
  // Split-KV decode form (DEC): one query token per sequence, q [B, h, d];
  // the g query heads of a KV head are the rows, one workgroup per
  // (sequence, KV head, split of chunk keys), K/V contiguous [B, h_kv, s_max,
  // d] or paged; the unnormalised state goes to part_o [B, h, max_splits, d],
  // part_m, part_l [B, h, max_splits] (natural-log units); seq_k holds the
  // key counts.
  float* part_o;
  float* part_m;
  float* part_l;
  int chunk, max_splits, s_max;
  // Paged forms with kPool32: bytes of one K (or V) pool (under 4 GB) and of
  // one page of it.
  uint32_t pool_bytes, page_bytes;
  // Optional launch order of the sequences (longest context first), given
  // when the host knows the key counts; n_order = 0 means natural order.
  int n_order;
  uint16_t order[kMaxOrder];
  float v_scale;   // 8-bit K/V (DEC): V's tensor scale, applied to the split's O~
};

// OPT flags: kStagers = decode with staging waves (at most 4 row blocks);
// kPool32 = paged pool under 4 GB, addressed with 32-bit buffer offsets;
// kKV8 = K and V hold one OCP E4M3 byte per element (decode with staging
// waves, contiguous or kPool32): the loads read 8 codes where a 16-bit tile
// has a 16-byte chunk, and the codes are converted as they are stored to LDS
// (K to the query type, V to fp16; both exact), so the compute waves see the
// tiles of the 16-bit form.
constexpr int kStagers = 1;
constexpr int kPool32 = 2;
constexpr int kKV8 = 4;

template <int DT, bool CAUSAL, bool KMASK, bool PAGED, bool DEC, int OPT>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p) {
  using E = Elem<DT>;
  constexpr bool stagers = (OPT & kStagers) != 0;
  constexpr bool pool32 = (OPT & kPool32) != 0;
  constexpr bool kv8 = (OPT & kKV8) != 0;
  static_assert(!kv8 || (DEC && stagers && (!PAGED || pool32)), "8-bit K/V: decode with staging waves");
  constexpr uint32_t kEB = kv8 ? 1u : 2u;   // bytes per stored K/V element
  // Raw load of 8 K/V elements, and its 16-bit form for the LDS tiles.
  using KVRaw = std::conditional_t<kv8, u32x2, u32x4>;
  auto kv_load = [](__amdgpu_buffer_rsrc_t r, uint32_t byte_off) -> KVRaw {
    if constexpr (kv8) return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, 0));
    else return buffer_load16(r, byte_off);
  };
  auto k16 = [](KVRaw x) -> u32x4 {
    if constexpr (kv8) return cvt8<DT>(x);
    else return x;
  };
  static_assert(!PAGED || KMASK, "paged K/V are addressed through the key-bit path");
  static_assert(!stagers || DEC, "staging waves are a decode form (at most 4 row blocks)");
  static_assert(!pool32 || PAGED, "32-bit pool offsets are a paged form");
  // K of tile t lives in slot t % 2 (read in iteration t - 1), V of tile t in
  // slot t % 3 (read in iteration t + 1).
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKElems];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[3][kVElems];
  // Contiguous key-masked prefill: the tiles with a visible key, in order.
  constexpr bool kCompact = KMASK && !PAGED && !DEC;
  __shared__ uint16_t tile_list[kCompact ? kMaxListTiles : 1];
  __shared__ int wave_count[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int col = lane & 31;   // query row inside the wave's block
  const int half = lane >> 5;

  const int n_bk = p.B * p.h_kv;
  int bk = blockIdx.x % n_bk;
  int grp = p.n_grp - 1 - (int)(blockIdx.x / n_bk);
  int split = 0;
  if (DEC) {
    split = (int)(blockIdx.x % (unsigned)p.max_splits);
    bk = (int)(blockIdx.x / (unsigned)p.max_splits);
    grp = 0;
  } else if (PAGED && p.n_order > 0) {
    // Sequences in the given order (a workgroup's run time follows its
    // sequence's key count, so the longest go first); inside a sequence the
    // KV head varies fastest, as above, then the row group, heaviest first.
    const int per_seq = p.n_grp * p.h_kv;
    const int r = (int)(blockIdx.x / per_seq);
    const int rem = (int)(blockIdx.x - r * per_seq);
    bk = p.order[r] * p.h_kv + rem % p.h_kv;
    grp = p.n_grp - 1 - rem / p.h_kv;
  }
  const int b = bk / p.h_kv;
  const int kvh = bk - b * p.h_kv;

#ifdef ATTN_DEVICE_CHECKS
  // extents of the tensors (bytes; rows of Q, O and LSE)
  const size_t e_pool = PAGED ? ((size_t)p.num_pages << p.page_shift) * p.h_kv * kD * kEB : 0;
  const size_t e_kv = PAGED ? e_pool
                      : DEC ? (size_t)p.B * p.h_kv * p.s_max * kD * kEB
                            : (size_t)p.B * p.h_kv * p.T_k * kD * kEB;
  const size_t q_rows = DEC ? (size_t)p.B * p.h : PAGED ? (size_t)p.cu_q[p.B] * p.h : (size_t)p.B * p.h * p.T_q;
  const size_t e_bt = (size_t)p.B * p.max_pages * 4;
  const size_t part_rows = DEC ? (size_t)p.B * p.h * p.max_splits : 0;
#endif
  // Lengths of this sequence (uniform over the workgroup).
  int T_q = p.T_q, T_k = p.T_k, n_rb = p.n_rb, q_start = 0;
  int k_lo = 0;   // first key of the workgroup's range (DEC)
  if (DEC) {
    // Splits past the sequence write nothing; the merge counts the valid
    // ones from the same key count.
    const int s_raw = ATTN_IN_RANGE(p.seq_k + b, 4, p.seq_k, (size_t)p.B * 4, kSitePreLens) ? p.seq_k[b] : 0;
    if (s_raw <= 0) return;
    if (split >= min(p.max_splits, (s_raw + p.chunk - 1) / p.chunk)) return;
    const int s_len = min(s_raw, PAGED ? p.max_pages << p.page_shift : p.s_max);
    k_lo = split * p.chunk;
    const int k_hi = split == p.max_splits - 1 ? s_len : min(s_len, k_lo + p.chunk);
    T_k = max(0, k_hi - k_lo);   // keys counted from k_lo
  } else if (PAGED) {
    const bool lens_ok = ATTN_IN_RANGE(p.cu_q + b, 8, p.cu_q, ((size_t)p.B + 1) * 4, kSitePreLens) &&
                         ATTN_IN_RANGE(p.seq_k + b, 4, p.seq_k, (size_t)p.B * 4, kSitePreLens);
    q_start = lens_ok ? p.cu_q[b] : 0;
    T_q = lens_ok ? min(p.cu_q[b + 1] - q_start, p.T_q) : 0;
    T_k = lens_ok ? min(p.seq_k[b], p.max_pages << p.page_shift) : 0;
    n_rb = p.g * ((T_q + kRows - 1) / kRows);
    if (grp * kWaves >= n_rb) return;   // whole workgroup past this sequence's rows
  }

  const int rb = grp * kWaves + wave;
  const bool wave_valid = rb < n_rb;
  // DEC: the rows are the group's heads (T_q = g), head = the first of them.
  const int qblk = DEC ? rb : rb / p.g;
  const int head = DEC ? kvh * p.g : kvh * p.g + (rb - qblk * p.g);
  const int q0 = qblk * kRows;
  const int off = T_k - T_q;   // >= 0 when causal (bottom-right alignment)
  const int qrow = q0 + col;
  const int row_last_w = min(T_q - 1, q0 + kRows - 1);

  const int rb_last = min(grp * kWaves + kWaves - 1, n_rb - 1);
  const int row_last_wg = min(T_q - 1, (rb_last / p.g) * kRows + kRows - 1);
  int n_tiles = (T_k + kBc - 1) / kBc;
  if (CAUSAL) n_tiles = min(n_tiles, (row_last_wg + off) / kBc + 1);
  // Last tile with a key this wave may see (-1: none).
  int last = wave_valid ? n_tiles - 1 : -1;
  if (CAUSAL && wave_valid) last = min(last, (row_last_w + off) / kBc);

  // Q row qrow of this wave's head: [B, h, T_q, d], or token-major
  // [total_q, h, d] when PAGED (row stride h * d); DEC: head + qrow of
  // [B, h, d].
  const int q_rstride = PAGED && !DEC ? p.h * kD : kD;
  u32x4 qf[8];
  {
    const int hq = wave_valid ? head : 0;
    const uint16_t* qbase = DEC     ? p.q + ((size_t)b * p.h + hq) * kD
                            : PAGED ? p.q + ((size_t)q_start * p.h + hq) * kD
                                    : p.q + (size_t)(b * p.h + hq) * T_q * kD;
    // (checked build: the rows this wave reads, head hq of rows 0 .. T_q - 1)
    const bool q_ok = !wave_valid || T_q <= 0 ||
                      ATTN_IN_RANGE(qbase, ((size_t)(T_q - 1) * q_rstride + kD) * 2, p.q, q_rows * kD * 2, kSitePreQ);
    const auto rq = make_rsrc(qbase, wave_valid && q_ok ? (uint32_t)T_q * q_rstride * 2 : 0u);
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = buffer_load16(rq, (uint32_t)(qrow * q_rstride + c * 16 + half * 8) * 2u);
  }

  const size_t kv_base = PAGED ? 0 : DEC ? ((size_t)bk * p.s_max + k_lo) * kD : (size_t)bk * T_k * kD;
  // (kPool32: the whole pools)
  uint32_t kv_range = PAGED ? (pool32 ? p.pool_bytes : 0u) : (uint32_t)T_k * kD * kEB;
  if (kv_range != 0 &&
      !(ATTN_IN_RANGE(reinterpret_cast<const uint8_t*>(p.k) + kv_base * kEB, kv_range, p.k, e_kv, kSitePreKV) &&
        ATTN_IN_RANGE(reinterpret_cast<const uint8_t*>(p.v) + kv_base * kEB, kv_range, p.v, e_kv, kSitePreKV)))
    kv_range = 0u;
  const auto rk = make_rsrc(reinterpret_cast<const uint8_t*>(p.k) + kv_base * kEB, kv_range);
  const auto rv = make_rsrc(reinterpret_cast<const uint8_t*>(p.v) + kv_base * kEB, kv_range);

  // Staging: 1024 16-byte chunks per tile for K and for V; chunk tid + 512 i
  // holds key chunk / 16, d-chunk chunk % 16.
  KVRaw kreg[2], vreg[2];
  // (unsigned: the tiles just past the end of the longest key range lie at
  // about 2^31 bytes, which the buffer range check turns into zeros)
  auto tile_byte = [&](int t, int i) {
    return ((uint32_t)(t * kBc + ((tid + kThreads * i) >> 4)) * kD + (uint32_t)(tid & 15) * 8u) * kEB;
  };
  // Per-lane loads that decide masking (block-table entries, key-mask bytes)
  // are range-checked buffer loads over the sequence's row: past its end
  // they read zero, so they need no branch, and the range test is applied
  // where the value is used. A branch around such a load would make the
  // compiler wait for it (and, loads retiring in order, for every tile load
  // issued before it) right where the branches join, before the products.
  const bool key_row_ok =
      !KMASK || (PAGED ? ATTN_IN_RANGE(p.bt + (size_t)b * p.max_pages, (size_t)p.max_pages * 4, p.bt, e_bt, kSitePreKeyRow)
                       : ATTN_IN_RANGE(p.key_mask + (size_t)b * T_k, (size_t)T_k, p.key_mask, (size_t)p.B * p.T_k,
                                       kSitePreKeyRow));
  const auto r_key = !KMASK ? make_rsrc(nullptr, 0u)
                     : PAGED ? make_rsrc(p.bt + (size_t)b * p.max_pages, key_row_ok ? (uint32_t)p.max_pages * 4u : 0u)
                             : make_rsrc(p.key_mask + (size_t)b * T_k, key_row_ok ? (uint32_t)T_k : 0u);
  // Paged: the block-table entry of staging row i of tile t, and the pool row
  // it gives; keys past T_k or on a page id outside the pool read as zeros.
  // Page ids are fetched one iteration before the K tile that needs them and
  // reused for the V tile one iteration later, so no tile load waits on a
  // block-table load.
  // kPool32: the rows a wave stages from a tile come in groups that lie on
  // one page (4 rows from a 4-aligned key for the compute waves, 16 from a
  // 16-aligned one for the staging waves; pages hold at least 16 keys and
  // ranges start 16-aligned), so those page ids are read with scalar loads
  // (the block table does not change during the kernel).
  const __attribute__((address_space(4))) int32_t* bt_row =
      (const __attribute__((address_space(4))) int32_t*)(PAGED ? p.bt + (size_t)b * p.max_pages : p.bt);
  auto page_of = [&](int t, int i) -> int {
    if (pool32) {   // rows 4 wave + 32 i + 0..3 of tile t
      const int idx = min((k_lo + t * kBc + 4 * wave + 32 * i) >> p.page_shift, p.max_pages - 1);
      return ATTN_IN_RANGE(p.bt + (size_t)b * p.max_pages + idx, 4, p.bt, e_bt, kSitePreTableRow) ? bt_row[idx] : -1;
    }
    const uint32_t key = (uint32_t)(k_lo + t * kBc + ((tid + kThreads * i) >> 4));
    return (int)__builtin_amdgcn_raw_buffer_load_b32(r_key, (int)((key >> p.page_shift) * 4u), 0, 0);
  };
  auto paged_row = [&](int t, int i, int page) -> long {
    const int key_l = t * kBc + ((tid + kThreads * i) >> 4);
    if (key_l >= T_k || page < 0 || page >= p.num_pages) return -1;
    const int key = k_lo + key_l;
    return (((long)page << p.page_shift) + (key & ((1 << p.page_shift) - 1))) * p.h_kv + kvh;
  };
  // kPool32: byte offset of this lane's chunk of staging row i of tile t on
  // page `page` (the wave's group offset, uniform, plus a per-lane constant);
  // past the pool's range (reads zeros) when the row is past T_k or the page
  // lies outside the pool.
  const uint32_t main_lane_off =
      ((uint32_t)(lane >> 4) * (uint32_t)p.h_kv + (uint32_t)kvh) * (kD * kEB) + (uint32_t)(tid & 15) * 8u * kEB;
  auto pool_off = [&](int t, int i, int page) -> uint32_t {
    const int g = t * kBc + 4 * wave + 32 * i;   // first key of the wave's 4 rows, counted from k_lo
    const bool ok = (uint32_t)page < (uint32_t)p.num_pages;
    const uint32_t slot0 = (uint32_t)(k_lo + g) & ((1u << p.page_shift) - 1u);
    const uint32_t go = ok ? (uint32_t)page * p.page_bytes + slot0 * (uint32_t)p.h_kv * (kD * kEB) : p.pool_bytes;
    return g + (lane >> 4) < T_k ? go + main_lane_off : 0xFFFFFFF0u;
  };
  int pg_k[2] = {-1, -1}, pg_v[2] = {-1, -1}, pg_n[2] = {-1, -1};
  auto load_k = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (PAGED && pool32) {
        kreg[i] = kv_load(rk, pool_off(t, i, pg_k[i]));
      } else if constexpr (PAGED && !kv8) {
        const long r = paged_row(t, i, pg_k[i]);
        kreg[i] = r >= 0 && ATTN_IN_RANGE(p.k + r * kD + (tid & 15) * 8, 16, p.k, e_pool, kSitePrePagedKV)
                      ? load16(p.k + r * kD + (tid & 15) * 8)
                      : u32x4{0u, 0u, 0u, 0u};
      } else {
        kreg[i] = kv_load(rk, tile_byte(t, i));
      }
    }
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (PAGED && pool32) {
        vreg[i] = kv_load(rv, pool_off(t, i, pg_v[i]));
      } else if constexpr (PAGED && !kv8) {
        const long r = paged_row(t, i, pg_v[i]);
        vreg[i] = r >= 0 && ATTN_IN_RANGE(p.v + r * kD + (tid & 15) * 8, 16, p.v, e_pool, kSitePrePagedKV)
                      ? load16(p.v + r * kD + (tid & 15) * 8)
                      : u32x4{0u, 0u, 0u, 0u};
      } else {
        vreg[i] = kv_load(rv, tile_byte(t, i));
      }
    }
  };
  auto store_k = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      store16(&lds_k[slot][((tid + kThreads * i) >> 4) * kKStr + (tid & 15) * 8], k16(kreg[i]));
  };
  // V tiles reach LDS in the element type of the PV product: fp16 in the
  // fp16 pass (bf16 inputs are converted here, exactly below 65536 in
  // magnitude, to +-inf from 65536 up), the input type in the fallback pass.
  // (8-bit V: codes straight to the pass's type; at most 448 in magnitude.)
  auto conv_v = [&](KVRaw x, auto pv16) -> u32x4 {
    if constexpr (kv8) {
      return cvt8<decltype(pv16)::value ? ATTN_DTYPE_F16 : DT>(x);
    } else {
      if constexpr (decltype(pv16)::value && DT == ATTN_DTYPE_BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = bf16x2_to_f16x2(x[e]);
      }
      return x;
    }
  };
  auto store_v = [&](int slot, auto pv16) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      store16(&lds_v[slot][((tid + kThreads * i) >> 4) * kVStr + (tid & 15) * 8], conv_v(vreg[i], pv16));
  };

  const int v_lane_off = (4 * half + ((lane & 15) >> 2)) * kVStr + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 acc[4];
  float m_ref = -INFINITY;
  float l_run = 0.f;
  float lr_run = 0.f;

  // S^T of one tile into s (K tile from LDS, Q from registers).
  auto qk = [&](const uint16_t* ks, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint16_t* kr = ks + (kb * 32 + col) * kKStr + half * 8;
      s[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < 8; ++c) s[kb] = E::mfma32(load16(kr + c * 16), qf[c], s[kb]);
    }
  };
  // Masking of tile t's scores where the tile needs it; every score of a
  // tile past the wave's last visible tile is masked, which makes the extra
  // pipeline iterations add exact zeros.
  auto mask = [&](int t, uint64_t kbits, f32x16 (&s)[2]) {
    const int kt = t * kBc;
    bool need = kt + kBc > T_k || t > last;
    if (CAUSAL) need = need || (kt + kBc - 1 > q0 + off);
    if (KMASK) need = need || (kbits != ~0ull);
    if (need) {
      // key offset ko = kb*32 + 8*(r/4) + 4*half + r%4 is visible when
      // ko - 4*half <= lim
      int lim = T_k - kt - 1;
      if (CAUSAL) lim = min(lim, qrow + off - kt);
      lim = t > last ? -1000 : lim - 4 * half;
      const uint32_t w0 = (uint32_t)kbits >> (4 * half);
      const uint32_t w1 = (uint32_t)(kbits >> 32) >> (4 * half);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = kb * 32 + (r >> 2) * 8 + (r & 3);
          bool vis = kc <= lim;
          if (KMASK) vis = vis && (((kb ? w1 : w0) >> (kc - kb * 32)) & 1u);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }
  };
  // Visible-key bits of tile t (KMASK): the key mask, or with PAGED the keys
  // whose block-table entry names a page of the pool. The per-lane value is
  // loaded early (key_raw) and turned into bits late (key_ballot, with the
  // range test), so the ballot's wait falls where the tile loads are awaited
  // anyway.
  auto key_raw = [&](int t) -> int {
    const uint32_t key = (uint32_t)(t * kBc + lane);
    return PAGED ? (int)__builtin_amdgcn_raw_buffer_load_b32(r_key, (int)(((k_lo + key) >> p.page_shift) * 4u), 0, 0)
                 : (int)__builtin_amdgcn_raw_buffer_load_b8(r_key, (int)key, 0, 0);
  };
  auto key_ballot = [&](int t, int raw) -> uint64_t {
    const bool in = t * kBc + lane < T_k;
    return __ballot(in && (PAGED ? (raw >= 0 && raw < p.num_pages) : raw != 0));
  };

  // Fully masked tiles are skipped: with a key mask, the pipeline below
  // walks the list of tiles that hold a visible key (position j -> tile
  // tile_at(j)); a skipped tile would only have added exact zeros. Each wave
  // scans a contiguous share of the tiles (the mask bytes of 8 tiles in
  // flight at a time), then the shares are concatenated in order.
  int n_vis = n_tiles;
  const bool use_list = kCompact && n_tiles <= kMaxListTiles;
  if (use_list) {
    uint16_t* found = lds_v[1];   // per-wave scratch; V slot 1 is first written below
    const int per = (n_tiles + kWaves - 1) / kWaves;
    const int t0 = wave * per;
    const int t1 = min(n_tiles, t0 + per);
    int cnt = 0;
    for (int tb = t0; tb < t1; tb += 8) {
      int raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = key_raw(tb + u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (tb + u < t1 && key_ballot(tb + u, raw[u]) != 0) {
          if (lane == 0) found[t0 + cnt] = (uint16_t)(tb + u);
          ++cnt;
        }
      }
    }
    if (lane == 0) wave_count[wave] = cnt;
    __syncthreads();
    int before = 0;
    n_vis = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = wave_count[w];
      before += w < wave ? c : 0;
      n_vis += c;
    }
    for (int i = lane; i < cnt; i += 64) tile_list[before + i] = found[t0 + i];
    __syncthreads();
  }
  // Positions past the list map to the tile past the last one: zeros, fully
  // masked.
  const int t_end = (T_k + kBc - 1) / kBc;
  auto tile_at = [&](int j) -> int {
    if (!use_list) return j;
    return j < n_vis ? (int)tile_list[j] : t_end;
  };

  // One pass over the key tiles. PV16: the PV product takes fp16 operands
  // (P rounded to fp16 -- 3 more significand bits than bf16 -- and V as
  // staged by store_v); with bf16 inputs the pass is run again with bf16
  // operands if a V value of magnitude 65536 or more was staged (fp16 cannot
  // hold it; it was staged as +-inf). Every wave of the workgroup takes the
  // same passes.
  auto pass = [&](auto pv16) {
  constexpr bool PV16 = decltype(pv16)::value;
  using EP = Elem<PV16 ? ATTN_DTYPE_F16 : DT>;
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  m_ref = -INFINITY;
  l_run = 0.f;
  lr_run = 0.f;
  f32x16 sc[2];     // scores of tile j
  u32x4 pp[4];      // P^T of tile j - 1
  uint64_t kbits = ~0ull;
#pragma unroll
  for (int i = 0; i < 4; ++i) pp[i] = u32x4{};
  sc[0] = f32x16{};
  sc[1] = f32x16{};

  if (n_vis > 0) {
    if (PAGED) {
      pg_k[0] = page_of(0, 0);
      pg_k[1] = page_of(0, 1);
      pg_v[0] = pg_k[0];
      pg_v[1] = pg_k[1];
    }
    load_k(tile_at(0));
    load_v(tile_at(0));
    store_k(0);
    store_v(0, pv16);
    if (n_vis > 1) {
      if (PAGED) {
        pg_k[0] = page_of(1, 0);
        pg_k[1] = page_of(1, 1);
      }
      load_k(tile_at(1));
      store_k(1);
    }
    if (KMASK) kbits = key_ballot(tile_at(0), key_raw(tile_at(0)));
  }
  if (PAGED) {
    // pages of tile 1 for V(1) and of tile 2 for K(2), used in iteration 0
    pg_v[0] = page_of(1, 0);
    pg_v[1] = page_of(1, 1);
    pg_k[0] = page_of(2, 0);
    pg_k[1] = page_of(2, 1);
  }
  // V slot 2 is read (with P = 0) in the first iteration.
  for (int i = tid; i < kVElems / 8; i += kThreads) store16(&lds_v[2][i * 8], u32x4{});
  __syncthreads();
  // kStagers (decode with at most 128 heads, launched only for n_rb <= 4):
  // waves 4-7 have no rows and stage every K/V tile of the main loop; waves
  // 0-3 only compute.
  if (stagers && wave >= 4) {
    // The pair stored in iteration j, K(j+2) and V(j+1), was loaded in
    // iteration j-2 into one of two register sets, so each CU keeps two tile
    // pairs (64 KB) of loads in flight instead of one. Each lane holds 16-byte
    // chunk st + 256 i of a tile (row st / 16 + 16 i). Paged: the pages of the
    // loads issued in iteration j are looked up in iteration j-1, before that
    // iteration's tile loads; loads retire in order, so waiting for the
    // lookups waits only for loads issued before them, i.e. the pair stored in
    // iteration j. The loop is unrolled by two so that the register sets and
    // the page sets have fixed registers (a copy of a pending load would wait
    // for it). Loads issued for tiles past the end are never stored.
    const int st = tid - 4 * 64;
    __syncthreads();   // the other waves' reads of K(0), below
    auto s_row = [&](int i) { return (st >> 4) + 16 * i; };
    auto s_page = [&](int t, int i) -> int {
      const uint32_t key = (uint32_t)(k_lo + t * kBc + s_row(i));
      return (int)__builtin_amdgcn_raw_buffer_load_b32(r_key, (int)((key >> p.page_shift) * 4u), 0, 0);
    };
    // kPool32: staging group i of a tile (rows 16 i .. 16 i + 15 of it, from a
    // 16-aligned key) lies on one page, so its page id and its byte offset in
    // the pool are the same for every staging lane. The page ids are read
    // with scalar loads one step before use, and the group's offset is added
    // to a per-lane
    // constant; a group past the keys or on a page outside the pool gets the
    // pool's size, past the range, which reads zeros.
    const uint32_t lane_off =
        ((uint32_t)(st >> 4) * (uint32_t)p.h_kv + (uint32_t)kvh) * (kD * kEB) + (uint32_t)(st & 15) * 8u * kEB;
    auto grp_page = [&](int t, int i) -> int {   // first key of the group: t * kBc + 16 i from k_lo
      const int idx = min((k_lo + t * kBc + 16 * i) >> p.page_shift, p.max_pages - 1);
      return ATTN_IN_RANGE(p.bt + (size_t)b * p.max_pages + idx, 4, p.bt, e_bt, kSitePreTableRow) ? bt_row[idx] : -1;
    };
    auto grp_off = [&](int t, int i, int page) -> uint32_t {
      const int g = t * kBc + 16 * i;
      const bool ok = g < T_k && (uint32_t)page < (uint32_t)p.num_pages;
      const uint32_t slot0 = (uint32_t)(k_lo + g) & ((1u << p.page_shift) - 1u);
      return ok ? (uint32_t)page * p.page_bytes + slot0 * (uint32_t)p.h_kv * (kD * kEB) : p.pool_bytes;
    };
    // Paged: a chunk whose row is past the keys or on a page outside the pool
    // reads zeros through an offset past the pool's range (kPool32), or, with
    // 64-bit addressing, loads pool row 0 and is stored as zeros (bit i (K) and
    // 4 + i (V) of ok[u] mark the valid chunks). Neither form branches: a
    // conditional load would make the compiler count it as possibly not
    // issued and wait for later loads too.
    auto s_load = [&](const uint16_t* pool, const decltype(rk)& r, int t, int i, int page, uint32_t& ok,
                      int bit) -> KVRaw {
      if constexpr (!PAGED) {
        return kv_load(r, ((uint32_t)(t * kBc + s_row(i)) * kD + (uint32_t)(st & 15) * 8u) * kEB);
      } else {
        const int key_l = t * kBc + s_row(i);
        if constexpr (pool32) {
          return kv_load(r, key_l < T_k ? grp_off(t, i, page) + lane_off : 0xFFFFFFF0u);
        } else {
          const bool valid = key_l < T_k && page >= 0 && page < p.num_pages;
          const long row =
              valid ? (((long)page << p.page_shift) + ((k_lo + key_l) & ((1 << p.page_shift) - 1))) * p.h_kv + kvh
                    : 0;
          ok |= valid ? 1u << bit : 0u;
          return ATTN_IN_RANGE(pool + row * kD + (st & 15) * 8, 16, pool, e_pool, kSitePrePagedKV)
                     ? load16(pool + row * kD + (st & 15) * 8)
                     : u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    KVRaw sk[2][4], sv[2][4];
    uint32_t ok[2] = {0u, 0u};
    int pgk[2][4], pgv[2][4];   // paged: pages of the K and V loads of the next two iterations
    auto lookup = [&](int u, int tk, int tv) {
      if (!PAGED) return;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pgk[u][i] = pool32 ? grp_page(tk, i) : s_page(tk, i);
        pgv[u][i] = pool32 ? grp_page(tv, i) : s_page(tv, i);
      }
    };
    auto issue = [&](int u, int tk, int tv, int pu) {
      ok[u] = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sk[u][i] = s_load(p.k, rk, tk, i, PAGED ? pgk[pu][i] : 0, ok[u], i);
        sv[u][i] = s_load(p.v, rv, tv, i, PAGED ? pgv[pu][i] : 0, ok[u], 4 + i);
      }
    };
    auto put = [&](int j, int u) {
      const KVRaw zero = {};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool as_is = !PAGED || pool32;
        store16(&lds_k[j & 1][s_row(i) * kKStr + (st & 15) * 8], k16(as_is || (ok[u] >> i & 1u) ? sk[u][i] : zero));
        store16(&lds_v[(j + 1) % 3][s_row(i) * kVStr + (st & 15) * 8],
                conv_v(as_is || (ok[u] >> (4 + i) & 1u) ? sv[u][i] : zero, pv16));
      }
    };
    // The pairs stored in iterations 0 and 1, with the pages of iteration 0's
    // loads looked up between them: the loads then stand in the order of the
    // steady state (pair, pages, pair), so the waits the compiler derives for
    // the loop hold on entry too.
    // (The scheduling fences keep the compiler from moving tile loads above
    // the lookups issued before them.)
    lookup(1, 2, 1);
    issue(0, 2, 1, 1);
    lookup(1, 3, 2);
    lookup(0, 4, 3);
    __builtin_amdgcn_sched_barrier(0);
    issue(1, 3, 2, 1);
    auto step = [&](int j, int u) {
      put(j, u);
      if (pool32) {
        // scalar lookups after the tile loads: the wait for them, before the
        // next step's loads, then also covers only loads already done
        issue(u, j + 4, j + 3, u);
        lookup(u ^ 1, j + 5, j + 4);
      } else {
        lookup(u ^ 1, j + 5, j + 4);
        __builtin_amdgcn_sched_barrier(0);
        issue(u, j + 4, j + 3, u);
      }
      __syncthreads();
    };
    // One barrier per iteration j = 0 .. n_tiles, as in the main loop.
    int j = 0;
    for (; j + 1 <= n_tiles; j += 2) {
      step(j, 0);
      step(j + 1, 1);
    }
    if (j <= n_tiles) {
      put(j, 0);
      __syncthreads();
    }
    return;
  }
  qk(lds_k[0], sc);
  // Iteration 0 overwrites K(0)'s slot with K(2) before its barrier: every
  // wave's reads of K(0) must be done first.
  __syncthreads();

  float alpha = 1.f;   // rescale of O~ decided by the previous softmax
  for (int j = 0; j <= n_vis; ++j) {
    // Tiles past the end load as zeros; the slots they go to are free, so the
    // loads and stores need no conditions and the iteration stays one block
    // from the rescale below to the barrier.
    if (!stagers) {
      load_k(tile_at(j + 2));
      load_v(tile_at(j + 1));
      if (PAGED) {
        pg_n[0] = page_of(j + 3, 0);
        pg_n[1] = page_of(j + 3, 1);
      }
    }
    int kraw = 0;
    const int t_kb = tile_at(j + 1);
    if (KMASK) kraw = key_raw(t_kb);
    // O~ still holds PV(j-2) at the old reference; PV(j-1) below uses the
    // weights of the current one.
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    }

    f32x16 sn[2];
    u32x4 pn[4];
    mask(tile_at(j), kbits, sc);
    {
      // Steady state: the 32 MFMAs of PV(j-1) and QK(j+1) in 8 slices of 4,
      // each slice carrying a share of the softmax VALU work of tile j, with
      // the MFMA operands of a slice read from LDS one slice ahead.
      const uint16_t* vs = lds_v[(j + 2) % 3];
      const uint16_t* ks = lds_k[(j + 1) & 1];
      auto read_v = [&](int cc, u32x4 (&va)[4]) {
        const uint16_t* vr = vs + cc * 16 * kVStr + v_lane_off;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const u32x2 lo = lds_read_tr16(vr + db * 32);
          const u32x2 hi = lds_read_tr16(vr + 8 * kVStr + db * 32);
          va[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      };
      auto read_k = [&](int c2, u32x4 (&kf)[4]) {
        // fragments c = 2*c2, 2*c2+1 of both 32-key blocks
#pragma unroll
        for (int i = 0; i < 4; ++i)
          kf[i] = load16(ks + ((i & 1) * 32 + col) * kKStr + half * 8 + (2 * c2 + (i >> 1)) * 16);
      };
      u32x4 fa[4], fb[4];
      float mx, base, rs = 0.f;
      // slice 0: PV chunk 0 | row maxima
      read_v(0, fa);
      // one chain of three-operand maxima (max(max(m, a), b) is one v_max3)
      mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, sc[0][r]), sc[1][r]);
      read_v(1, fb);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = EP::mfma32(fa[db], pp[0], acc[db]);
      __builtin_amdgcn_sched_barrier(0);
      // slice 1: PV chunk 1 | reference update, exps of block 0 rows 0-7
      read_v(2, fa);
      {
        const float mr = max_halves(mx) * p.c;
        const bool move = mr > m_ref + kTau;
        alpha = move ? fast_exp2(m_ref - mr) : 1.f;
        m_ref = move ? mr : m_ref;
        l_run *= alpha;
        lr_run *= alpha;
        base = m_ref == -INFINITY ? 0.f : m_ref;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = EP::mfma32(fb[db], pp[1], acc[db]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        sc[0][r] = fast_exp2(__builtin_fmaf(sc[0][r], p.c, -base));
        rs += sc[0][r];
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 2: PV chunk 2 | exps of block 0 rows 8-15
      read_v(3, fb);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = EP::mfma32(fa[db], pp[2], acc[db]);
#pragma unroll
      for (int r = 8; r < 16; ++r) {
        sc[0][r] = fast_exp2(__builtin_fmaf(sc[0][r], p.c, -base));
        rs += sc[0][r];
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 3: PV chunk 3 | exps of block 1 rows 0-7
      read_k(0, fa);
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = EP::mfma32(fb[db], pp[3], acc[db]);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        sc[1][r] = fast_exp2(__builtin_fmaf(sc[1][r], p.c, -base));
        rs += sc[1][r];
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 4: QK fragments 0-1 | exps of block 1 rows 8-15
      read_k(1, fb);
      sn[0] = E::mfma32(fa[0], qf[0], f32x16{});
      sn[1] = E::mfma32(fa[1], qf[0], f32x16{});
      sn[0] = E::mfma32(fa[2], qf[1], sn[0]);
      sn[1] = E::mfma32(fa[3], qf[1], sn[1]);
#pragma unroll
      for (int r = 8; r < 16; ++r) {
        sc[1][r] = fast_exp2(__builtin_fmaf(sc[1][r], p.c, -base));
        rs += sc[1][r];
      }
      l_run += rs;
      __builtin_amdgcn_sched_barrier(0);
      // slices 5-7: QK fragments 2-7 | packing of P^T and the sum of p~
#pragma unroll
      for (int c2 = 1; c2 < 4; ++c2) {
        u32x4 (&cur)[4] = (c2 & 1) ? fb : fa;
        u32x4 (&nxt)[4] = (c2 & 1) ? fa : fb;
        if (c2 < 3) read_k(c2 + 1, nxt);
        sn[0] = E::mfma32(cur[0], qf[2 * c2], sn[0]);
        sn[1] = E::mfma32(cur[1], qf[2 * c2], sn[1]);
        sn[0] = E::mfma32(cur[2], qf[2 * c2 + 1], sn[0]);
        sn[1] = E::mfma32(cur[3], qf[2 * c2 + 1], sn[1]);
        if (c2 == 1) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const int r0 = cc * 8;
            pn[cc] = u32x4{EP::pack2(sc[0][r0 + 0], sc[0][r0 + 1]), EP::pack2(sc[0][r0 + 2], sc[0][r0 + 3]),
                           EP::pack2(sc[0][r0 + 4], sc[0][r0 + 5]), EP::pack2(sc[0][r0 + 6], sc[0][r0 + 7])};
          }
        } else if (c2 == 2) {
#pragma unroll
          for (int cc = 2; cc < 4; ++cc) {
            const int r0 = (cc - 2) * 8;
            pn[cc] = u32x4{EP::pack2(sc[1][r0 + 0], sc[1][r0 + 1]), EP::pack2(sc[1][r0 + 2], sc[1][r0 + 3]),
                           EP::pack2(sc[1][r0 + 4], sc[1][r0 + 5]), EP::pack2(sc[1][r0 + 6], sc[1][r0 + 7])};
          }
        } else {
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
            lr_run = EP::add_pair(pn[cc][3], EP::add_pair(pn[cc][2], EP::add_pair(pn[cc][1], EP::add_pair(pn[cc][0], lr_run))));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) pp[i] = pn[i];
    sc[0] = sn[0];
    sc[1] = sn[1];
    if (KMASK) kbits = key_ballot(t_kb, kraw);
    if (!stagers) {
      if (PAGED) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          pg_v[i] = pg_k[i];
          pg_k[i] = pg_n[i];
        }
      }
      store_k(j & 1);
      store_v((j + 1) % 3, pv16);
    }
    __syncthreads();
  }
  };

  pass(std::true_type{});
  if constexpr (DT == ATTN_DTYPE_BF16 && !kv8) {
    // A staged V value fp16 cannot hold was stored as +-inf. Every staged V
    // row enters the PV product of every computing wave (a key a wave does
    // not see has weight 0, and 0 * inf is NaN), and O~ is otherwise finite
    // for finite inputs (at most 65280 * 2^kTau per key), so a non-finite O~
    // in any wave means such a value, or a non-finite input. The workgroup
    // then runs the pass again with bf16 operands (all waves take the same
    // decision; with non-finite inputs the second pass gives what they give).
    if (__syncthreads_or(any_nonfinite(acc))) pass(std::false_type{});
  }
  if (stagers && wave >= 4) return;
  if (!wave_valid || qrow >= T_q) return;
  const float l_tot = sum_halves(l_run);
  const float lr_tot = sum_halves(lr_run);
  if (DEC) {
    // Partial state of the split at the reference m: O~ accumulated the
    // rounded weights, so it is scaled by l / l~ to pair with l (the merge
    // divides the combined O~ by the combined l), and, with 8-bit V, by V's
    // tensor scale. No visible key: m = -inf, l = 0, O~ = 0.
    const bool none = l_tot == 0.f;
    const float rs = none ? 0.f : l_tot / lr_tot * (kv8 ? p.v_scale : 1.f);
    const size_t hs = ((size_t)b * p.h + head + qrow) * p.max_splits + split;
    float* po = p.part_o + hs * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        if (ATTN_IN_RANGE(po + db * 32 + g4 * 8 + half * 4, 16, p.part_o, part_rows * kD * 4, kSitePrePartO))
          *reinterpret_cast<f32x4*>(po + db * 32 + g4 * 8 + half * 4) =
              f32x4{acc[db][g4 * 4 + 0] * rs, acc[db][g4 * 4 + 1] * rs, acc[db][g4 * 4 + 2] * rs,
                    acc[db][g4 * 4 + 3] * rs};
    if (half == 0 && ATTN_IN_RANGE(p.part_m + hs, 4, p.part_m, part_rows * 4, kSitePrePartML) &&
        ATTN_IN_RANGE(p.part_l + hs, 4, p.part_l, part_rows * 4, kSitePrePartML)) {
      p.part_m[hs] = none ? -INFINITY : m_ref * kLn2;
      p.part_l[hs] = l_tot;
    }
    return;
  }
  bool empty = l_tot == 0.f;
  if (!PAGED && p.row_mask != nullptr &&
      ATTN_IN_RANGE(p.row_mask + (size_t)b * T_q + qrow, 1, p.row_mask, (size_t)p.B * p.T_q, kSitePreRowMask))
    empty = empty || p.row_mask[(size_t)b * T_q + qrow] == 0;
  const float inv = empty ? 0.f : 1.f / lr_tot;
  const size_t orow = PAGED ? (size_t)(q_start + qrow) * p.h + head : (size_t)(b * p.h + head) * T_q + qrow;
  uint16_t* op = p.o + orow * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + half * 4;
      float v0 = acc[db][g4 * 4 + 0] * inv, v1 = acc[db][g4 * 4 + 1] * inv;
      float v2 = acc[db][g4 * 4 + 2] * inv, v3 = acc[db][g4 * 4 + 3] * inv;
      if (empty) v0 = v1 = v2 = v3 = 0.f;
      if (ATTN_IN_RANGE(op + d, 8, p.o, q_rows * kD * 2, kSitePreO))
        store8(op + d, u32x2{E::pack2(v0, v1), E::pack2(v2, v3)});
    }
  }
  if (p.lse != nullptr && half == 0 && ATTN_IN_RANGE(p.lse + orow, 4, p.lse, q_rows * 4, kSitePreLse))
    p.lse[orow] = empty ? -INFINITY : (m_ref + fast_log2(l_tot)) * kLn2;
}

template <int DT, bool CAUSAL, bool KMASK, bool PAGED>
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.n_grp * p.B * p.h_kv));
  if (PAGED && p.pool_bytes != 0)
    hipLaunchKernelGGL((prefill_kernel<DT, CAUSAL, KMASK, PAGED, false, PAGED ? kPool32 : 0>), grid, dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<DT, CAUSAL, KMASK, PAGED, false, 0>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// Split-KV decode on the prefill kernel (paged launches take the key-bit
// path for page ids outside the pool). 8-bit K/V: staging waves only (at
// most 128 heads), contiguous or with 32-bit pool offsets.
template <int DT, bool PAGED, bool KV8>
hipError_t launch_decode_rows(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((long)p.B * p.h_kv * p.max_splits));
  const bool stg = p.n_rb <= 4;
  if constexpr (KV8) {
    if (!stg || (PAGED && p.pool_bytes == 0)) return hipErrorInvalidValue;
    if constexpr (PAGED)
      hipLaunchKernelGGL((prefill_kernel<DT, false, true, true, true, kStagers | kPool32 | kKV8>), grid,
                         dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((prefill_kernel<DT, false, false, false, true, kStagers | kKV8>), grid, dim3(kThreads), 0,
                         stream, p);
  } else if constexpr (PAGED) {
    if (p.pool_bytes != 0) {
      if (stg)
        hipLaunchKernelGGL((prefill_kernel<DT, false, true, true, true, kStagers | kPool32>), grid, dim3(kThreads), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((prefill_kernel<DT, false, true, true, true, kPool32>), grid, dim3(kThreads), 0, stream, p);
    } else if (stg) {
      hipLaunchKernelGGL((prefill_kernel<DT, false, true, true, true, kStagers>), grid, dim3(kThreads), 0, stream, p);
    } else {
      hipLaunchKernelGGL((prefill_kernel<DT, false, true, true, true, 0>), grid, dim3(kThreads), 0, stream, p);
    }
  } else if (stg) {
    hipLaunchKernelGGL((prefill_kernel<DT, false, false, false, true, kStagers>), grid, dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((prefill_kernel<DT, false, false, false, true, 0>), grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t dispatch_prefill(const PrefillParams& p, bool causal, bool kmask, hipStream_t s) {
  if (causal) return kmask ? launch_prefill<DT, true, true, false>(p, s) : launch_prefill<DT, true, false, false>(p, s);
  return kmask ? launch_prefill<DT, false, true, false>(p, s) : launch_prefill<DT, false, false, false>(p, s);
}

// Paged launches take the key-bit path: keys on a page id outside the pool
// are excluded (masked), not read as zeros.
template <int DT>
hipError_t dispatch_prefill_paged(const PrefillParams& p, bool causal, hipStream_t s) {
  return causal ? launch_prefill<DT, true, true, true>(p, s) : launch_prefill<DT, false, true, true>(p, s);
}

// kPool32 when a pool [num_pages, page_size, h_kv, d] of elem_bytes-byte
// elements is under 4 GB, with room above it for the out-of-range offsets of
// invalid rows (the pool's size plus an in-page offset must not wrap); else
// the pool_bytes = 0 left by the caller selects the 64-bit addressing.
void set_pool32(PrefillParams& p, int num_pages, int h_kv, int page_shift, int elem_bytes = 2) {
  const uint64_t page_bytes = ((uint64_t)h_kv << page_shift) * kD * (uint64_t)elem_bytes;
  const uint64_t pool_bytes = (uint64_t)num_pages * page_bytes;
  if (pool_bytes + page_bytes <= 0xFFFFFF00ull) {
    p.pool_bytes = (uint32_t)pool_bytes;
    p.page_bytes = (uint32_t)page_bytes;
  }
}

PrefillParams common_params(const void* q, const void* k, const void* v, void* o, float* lse, int B, int h,
                            int h_kv, int T_q, int T_k, float scale) {
  PrefillParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
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
  p.v_scale = 1.f;
  return p;
}

}  // namespace

ATTN_DEFINE_CHECK_READER(prefill)

hipError_t prefill_fwd(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                       const uint8_t* row_mask, void* o, float* lse, int B, int h, int h_kv,
                       int T_q, int T_k, int dtype, float scale, int causal, hipStream_t stream) {
  PrefillParams p = common_params(q, k, v, o, lse, B, h, h_kv, T_q, T_k, scale);
  p.key_mask = key_mask;
  p.row_mask = row_mask;
  if (B == 0 || T_q == 0 || h == 0) return hipSuccess;
  if (dtype == ATTN_DTYPE_BF16) return dispatch_prefill<ATTN_DTYPE_BF16>(p, causal != 0, key_mask != nullptr, stream);
  return dispatch_prefill<ATTN_DTYPE_F16>(p, causal != 0, key_mask != nullptr, stream);
}

// Variable-length prefill against a paged KV cache: T_q is the largest query
// count of the batch (it sizes the grid; workgroups past a sequence's rows
// exit at once), T_k the largest key count the block table can address.
hipError_t prefill_paged(const void* q, const int32_t* cu_seqlens_q, int max_q, const void* k_pool,
                         const void* v_pool, const int32_t* block_table, const int32_t* seq_lens_k,
                         const int32_t* seq_lens_k_host, int B, int h, int h_kv, int page_shift, int max_pages,
                         int num_pages, void* o, float* lse, int dtype, float scale, int causal,
                         hipStream_t stream) {
  PrefillParams p = common_params(q, k_pool, v_pool, o, lse, B, h, h_kv, max_q, max_pages << page_shift, scale);
  if (seq_lens_k_host != nullptr && B <= kMaxOrder) {
    // Longest context first (stable), so the longest workgroups start first.
    int idx[kMaxOrder];
    for (int i = 0; i < B; ++i) idx[i] = i;
    std::stable_sort(idx, idx + B, [&](int a, int c) { return seq_lens_k_host[a] > seq_lens_k_host[c]; });
    for (int i = 0; i < B; ++i) p.order[i] = (uint16_t)idx[i];
    p.n_order = B;
  }
  p.cu_q = cu_seqlens_q;
  p.seq_k = seq_lens_k;
  p.bt = block_table;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  p.page_shift = page_shift;
  set_pool32(p, num_pages, h_kv, page_shift);
  if (B == 0 || max_q == 0 || h == 0) return hipSuccess;
  if (dtype == ATTN_DTYPE_BF16) return dispatch_prefill_paged<ATTN_DTYPE_BF16>(p, causal != 0, stream);
  return dispatch_prefill_paged<ATTN_DTYPE_F16>(p, causal != 0, stream);
}

// Split-KV decode with the query heads of a group as the MFMA rows: the
// stage-1 producer for groups of more than 16 heads (up to 256, one wave per
// 32 heads). page_shift < 0 means contiguous K/V [B, h_kv, s_max, d].
// kv8: K and V are E4M3 codes with tensor scales k_scale and v_scale (at most
// 128 heads per KV head; paged pools must fit 32-bit offsets, see
// decode_rows_fp8_supported).
hipError_t decode_split_rows(const void* q, const void* k, const void* v, const int32_t* block_table,
                             int max_pages, int page_shift, int num_pages, const int32_t* seq_lens, int s_max,
                             int B, int h, int h_kv, int chunk_keys, int max_splits, int dtype, float scale,
                             float* part_o, float* part_m, float* part_l, hipStream_t stream, bool kv8,
                             float k_scale, float v_scale) {
  PrefillParams p = common_params(q, k, v, nullptr, nullptr, B, h, h_kv, h / h_kv, 0, scale);
  p.n_rb = (p.g + kRows - 1) / kRows;
  p.n_grp = 1;
  p.seq_k = seq_lens;
  p.bt = block_table;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  p.page_shift = page_shift;
  p.part_o = part_o;
  p.part_m = part_m;
  p.part_l = part_l;
  p.chunk = chunk_keys;
  p.max_splits = max_splits;
  p.s_max = s_max;
  if (kv8) {
    p.c *= k_scale;   // scores (q . k_code) k_scale, in the one multiply by scale log2(e)
    p.v_scale = v_scale;
  }
  const bool paged = block_table != nullptr;
  if (paged) set_pool32(p, num_pages, h_kv, page_shift, kv8 ? 1 : 2);
  if (B == 0 || h == 0) return hipSuccess;
  const bool bf = dtype == ATTN_DTYPE_BF16;
  if (kv8) {
    if (bf) return paged ? launch_decode_rows<ATTN_DTYPE_BF16, true, true>(p, stream)
                         : launch_decode_rows<ATTN_DTYPE_BF16, false, true>(p, stream);
    return paged ? launch_decode_rows<ATTN_DTYPE_F16, true, true>(p, stream)
                 : launch_decode_rows<ATTN_DTYPE_F16, false, true>(p, stream);
  }
  if (bf) return paged ? launch_decode_rows<ATTN_DTYPE_BF16, true, false>(p, stream)
                       : launch_decode_rows<ATTN_DTYPE_BF16, false, false>(p, stream);
  return paged ? launch_decode_rows<ATTN_DTYPE_F16, true, false>(p, stream)
               : launch_decode_rows<ATTN_DTYPE_F16, false, false>(p, stream);
}

// Whether decode_split_rows takes 8-bit K/V of this shape: staging waves
// (g <= 128) and, paged, a pool that 32-bit offsets address.
bool decode_rows_fp8_supported(int g, bool paged, int num_pages, int h_kv, int page_shift) {
  if (g > 4 * kRows) return false;
  if (!paged) return true;
  PrefillParams p = {};
  set_pool32(p, num_pages, h_kv, page_shift, 1);
  return p.pool_bytes != 0;
}

}  // namespace attn
