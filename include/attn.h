/*
 * attn.h -- C ABI of libattn.so: exact scaled-dot-product attention computed
 * tile by tile with the online-softmax (m, l, O~) recurrence on AMD Instinct
 * MI355X (gfx950). The score matrix never reaches device memory.
 *
 * The operations follow four web pages:
 *  [NA] "Naive attention and the online softmax" (mlinterviewnotes.com,
 *       inference course 03-01)
 *  [OR] "The Online Softmax Recurrence" (inferenceinterviews.com)
 *  [DA] "Decode attention: FlashDecoding, split-K, paged kernels"
 *       (mlinterviewnotes.com, inference course 03-03)
 *  [MI] "Merge normalized attention without averaging tile outputs"
 *       (study.greatitself.com)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Layouts are row-major and contiguous. Element types: dtype 0 = IEEE fp16,
 *   1 = bfloat16 for Q/K/V/O; statistics, partials and LSE are always fp32
 *   ([NA] section "What has to be fp32"; [OR] section "Where it breaks").
 * - Every pointer except *_host arguments is a device pointer owned by the
 *   caller. The library allocates no device memory and keeps no state apart
 *   from a per-thread error message.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream). Nothing synchronises.
 * - GQA: query head i reads KV head i / g with g = h / h_kv ([NA] opening
 *   section; [DA] section "Where GQA enters").
 * - LSE is the natural log-sum-exp m + ln(l) of the visible logits of a row
 *   ([NA] section "The state that gets passed around is the log-sum-exp").
 * - A row with no visible key gets an output of all-zero bits (+0.0) and
 *   LSE = -inf ([MI], last paragraph: zero output as the extension for a
 *   fully masked row).
 * - Return value: ATTN_OK, or an error code. Arguments are validated before
 *   anything is launched; on error nothing is launched and attn_last_error()
 *   describes the problem. Nothing aborts and no C++ exception crosses the
 *   ABI.
 * - Supported today: d_h = 128; dtype f16 or bf16; h a multiple of h_kv;
 *   paged KV with page_size a positive multiple of 16 ([DA], paged
 *   addressing: kernel block sizes are multiples of 16). Anything else
 *   returns ATTN_ERR_UNSUPPORTED.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_DTYPE_F16 0
#define ATTN_DTYPE_BF16 1

#define ATTN_OK 0
#define ATTN_ERR_INVALID 1     /* malformed argument (null pointer, negative size, ...) */
#define ATTN_ERR_UNSUPPORTED 2 /* well-formed but outside the support matrix */
#define ATTN_ERR_HIP 3         /* the HIP runtime rejected a launch */

/*
 * Prefill: O = softmax(scale * Q K^T restricted to visible keys) V, per
 * (batch, query head, query row), with the per-row LSE.
 * [NA] opening section (shapes Q [h,T,d_h], K/V [h_kv,T,d_h]), sections (3)
 * "The online recurrence" and "Extending the recurrence to the output"
 * (one pass over key tiles, divide once at the end).
 *
 *   q        [B, h, T_q, d_h]      dtype
 *   k, v     [B, h_kv, T_k, d_h]   dtype
 *   key_mask [B, T_k] uint8 or NULL; nonzero = the key may be attended.
 *   row_mask [B, T_q] uint8 or NULL; zero = every key of that query row is
 *            masked (the row gets the zero output).
 *   o        [B, h, T_q, d_h]      dtype (written)
 *   lse      [B, h, T_q] fp32 or NULL (written if not NULL)
 *   scale    multiplies Q K^T before masking (normally 1/sqrt(d_h)).
 *   causal   nonzero: query t sees key j iff j <= t + T_k - T_q (aligned to
 *            the bottom-right corner); requires T_q <= T_k.
 * Visible = causal condition AND key_mask AND row_mask. Masked keys are
 * excluded, never given a finite stand-in value ([MI], paragraph on fully
 * masked tiles).
 */
int attn_prefill_fwd(const void* q, const void* k, const void* v,
                     const uint8_t* key_mask, const uint8_t* row_mask,
                     void* o, float* lse,
                     int B, int h, int h_kv, int T_q, int T_k, int d_h,
                     int dtype, float scale, int causal, void* stream);

/*
 * Prefill of new tokens against a paged KV cache, variable length (chunked
 * prefill in a serving batch): sequence b has T_q,b new query tokens, which
 * are the last T_q,b positions of its T_k,b-token context; query t attends
 * to keys j <= t + T_k,b - T_q,b when causal (bottom-right alignment), to
 * all T_k,b keys otherwise. [DA] opening section (the launcher packs the
 * query tokens of many sequences, with the g heads of a KV head, into
 * query-parallel blocks) and section "Where GQA enters" (a chunked-prefill
 * request in a mixed batch runs the query-parallel path over the paged
 * cache; the block-table addressing); the arithmetic is that of
 * attn_prefill_fwd ([NA] section "The online recurrence").
 *
 *   q            [total_q, h, d_h] dtype, token-major: the rows of sequence b
 *                are cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1.
 *   cu_seqlens_q [B + 1] int32 device, non-decreasing, cu_seqlens_q[0] = 0.
 *   max_q        host upper bound of every T_q,b; it sizes the grid. Rows
 *                past max_q of a longer sequence are not computed.
 *   k_pool, v_pool  [num_pages, page_size, h_kv, d_h] dtype.
 *   block_table  [B, max_pages] int32 device; key j of sequence b is slot
 *                j % page_size of page block_table[b][j / page_size]. A page
 *                id outside [0, num_pages) excludes its keys.
 *   seq_lens_k   [B] int32 device, T_k,b (at most max_pages * page_size; at
 *                least T_q,b when causal, else the first rows have no key).
 *   seq_lens_k_host  NULL, or the same counts on the host: then (for B <= 512)
 *                the sequences are launched longest context first, which
 *                balances the GPU when the contexts differ; results do not
 *                depend on it.
 *   page_size    a power of two in [16, 65536].
 *   o            [total_q, h, d_h] dtype (written).
 *   lse          [total_q, h] fp32 (written) or NULL.
 * Rows with no visible key get +0.0 and LSE -inf. No key or row masks here.
 */
int attn_prefill_paged(const void* q, const int32_t* cu_seqlens_q, int max_q,
                       const void* k_pool, const void* v_pool, const int32_t* block_table,
                       const int32_t* seq_lens_k, const int32_t* seq_lens_k_host,
                       int B, int h, int h_kv, int d_h,
                       int page_size, int max_pages, int num_pages, int dtype, float scale,
                       int causal, void* o, float* lse, void* stream);

/*
 * Decode plan (host only, pure): choose the split-KV chunk length so the
 * stage-1 grid fills the GPU. [DA] sections "The grid" (the smallest split
 * count that fills the machine in one wave) and "SGLang: a split count
 * computed per sequence" (more splits for longer contexts).
 *
 *   seq_lens_host [B] host int32, the KV length of each sequence.
 *   num_cus       compute units of the device (256 on MI355X).
 *   chunk_keys    (out) keys per split: a multiple of 64, at least 64.
 *   max_splits    (out) ceil(max_b seq_lens[b] / chunk_keys), at least 1:
 *                 the split dimension of the partial buffers.
 * The split count of sequence b is n_b = ceil(seq_lens[b] / chunk_keys);
 * units = h_kv * sum_b n_b is at least num_cus whenever the keys allow it.
 *
 * The plan depends on the whole batch, so a sequence's output bits may change
 * with its companions; attn_decode_plan_fixed gives batch-invariant plans.
 */
int attn_decode_plan(int B, const int32_t* seq_lens_host, int h, int h_kv, int d_h,
                     int num_cus, int32_t* chunk_keys, int32_t* max_splits);

/*
 * Batch-invariant decode plan (host only, pure): a split length fixed by the
 * caller instead of derived from the batch. [DA] section "Split-K breaks
 * bitwise reproducibility" (fix the split tile, so that the split count of a
 * sequence is a function of its own length alone) and section "CUDA graphs
 * need the split count pinned" (a grid sized once for the longest sequence,
 * the active splits decided on the device).
 *
 *   seq_lens_host [B] host int32, the KV length of each sequence (>= 0).
 *   split_keys    keys per split, a positive multiple of 16 (e.g. 2048).
 *   chunk_keys    (out) = split_keys.
 *   max_splits    (out) = max(1, ceil(max_b seq_lens[b] / split_keys)), the
 *                 split dimension of the partial buffers and of the grid.
 * With this plan, split i of sequence b covers keys [i*split_keys,
 * (i+1)*split_keys) and the merge sums a row's splits in an order that
 * depends only on its own split count, so each sequence's output and LSE
 * bits are the same whatever other sequences share the call. A plan whose
 * max_splits would exceed 65535 (what attn_decode_split accepts) returns
 * ATTN_ERR_UNSUPPORTED; a split_keys that is not a positive multiple of 16
 * or a negative length returns ATTN_ERR_INVALID. Outputs are written only
 * on success.
 */
int attn_decode_plan_fixed(int B, const int32_t* seq_lens_host, int split_keys,
                           int32_t* chunk_keys, int32_t* max_splits);

/*
 * Decode stage 1 (split-KV, FlashDecoding): one query token per sequence;
 * the KV of sequence b is cut into contiguous slices of chunk_keys keys and
 * each slice emits an unnormalised partial state per query head.
 * [DA] opening section (split-K over keys, partial O~, m, l), section
 * "Segment length, and the early exit", section "Where GQA enters" (all g
 * query heads of a KV head share one read of the KV), and the paged
 * addressing that follows "What the merge costs".
 *
 *   q            [B, h, d_h] dtype
 *   k, v         contiguous: [B, h_kv, s_max, d_h] (block_table == NULL;
 *                may be NULL when s_max = 0: no key exists);
 *                paged: pools [num_pages, page_size, h_kv, d_h].
 *   block_table  NULL, or [B, max_pages] int32 physical page ids: key p of
 *                sequence b is slot p % page_size of page
 *                block_table[b * max_pages + p / page_size].
 *   num_pages    pages in each pool (paged only). A key whose page id lies
 *                outside [0, num_pages) is excluded, never dereferenced.
 *   seq_lens     [B] int32 device, KV length of each sequence. Must not
 *                exceed s_max (contiguous) or max_pages * page_size (paged);
 *                keys past that bound are never read. s_max and
 *                max_pages * page_size are at most 2^23 (else
 *                ATTN_ERR_UNSUPPORTED).
 *   chunk_keys   positive multiple of 16 (attn_decode_plan returns a
 *                multiple of 64).
 *   max_splits   split dimension of the partial buffers.
 *   part_o       [B, h, max_splits, d_h] fp32: O~_i = sum exp(x - m_i) v
 *   part_m       [B, h, max_splits] fp32: m_i, the reference maximum of
 *                split i in natural-log units (-inf for a split with no key)
 *   part_l       [B, h, max_splits] fp32: l_i = sum exp(x - m_i)
 * Split i of sequence b covers keys [i*chunk_keys, (i+1)*chunk_keys), the
 * last split (i = max_splits-1) also takes any keys beyond. Exactly the splits
 * i < n_b = min(max_splits, ceil(seq_lens[b]/chunk_keys)) are written; the
 * others are left untouched, and attn_merge_states never uses their contents
 * (it may load them, inside the [B, h, max_splits] buffers, before it knows
 * n_b).
 * (m_i, l_i, O~_i) is a state in the sense of [OR] section "The recurrence":
 * m_i is its reference point, and any reference gives the same merged
 * result. This library stores a reference at most 8 ln 2 below the largest
 * logit of the split (the reference moves only when that logit exceeds it
 * by more than 8 ln 2), so every weight exp(x - m_i) is at most 2^8.
 */
int attn_decode_split(const void* q, const void* k, const void* v,
                      const int32_t* block_table, int max_pages, int page_size, int num_pages,
                      const int32_t* seq_lens, int s_max,
                      int B, int h, int h_kv, int d_h,
                      int chunk_keys, int max_splits, int dtype, float scale,
                      float* part_o, float* part_m, float* part_l, void* stream);

/*
 * Decode stage 2: merge the split partials of each (sequence, head).
 * [DA] "Stage 2" reduction in section "Where GQA enters" (global maximum,
 * rescale each split's l and O~ by exp(m_i - max), sum, divide once, zero
 * when the total mass is zero); [MI] paragraph on merging disjoint tiles;
 * [NA] section "The base case is a NaN factory" (an empty state never
 * produces NaN).
 *
 *   part_o/part_m/part_l  as written by attn_decode_split.
 *   seq_lens     [B] int32 device; with chunk_keys it gives the valid split
 *                count n_b, computed exactly as attn_decode_split does, so
 *                producer and reducer agree ([DA] section "CUDA graphs need
 *                the split count pinned").
 *   o            [B, h, d_h] dtype (written); lse [B, h] fp32 or NULL.
 * A split with m_i = -inf or l_i = 0 is empty and contributes nothing.
 */
int attn_merge_states(const float* part_o, const float* part_m, const float* part_l,
                      const int32_t* seq_lens, int chunk_keys,
                      int B, int h, int max_splits, int d_h,
                      void* o, float* lse, int dtype, void* stream);

/*
 * Split-KV decode, both stages in one call: stage 1 as attn_decode_split
 * into the caller's partial buffers, then the merge as attn_merge_states,
 * both on `stream`, with the same arguments, results and empty-row rules.
 * [DA] opening section (split-K over keys, partial O~, m, l, then a
 * reduction of the partials) and section "CUDA graphs need the split count
 * pinned" (producer and reducer agree on the valid split count of each
 * sequence). With a fixed chunk_keys (attn_decode_plan_fixed) each
 * sequence's bits do not depend on the rest of the batch.
 *
 *   part_o/part_m/part_l  [B, h, max_splits, d_h] / [B, h, max_splits] fp32,
 *                caller-owned scratch; their contents on return are the
 *                split states.
 *   o            [B, h, d_h] dtype (written); lse [B, h] fp32 or NULL.
 * Errors as attn_decode_split; NULL partials or o: ATTN_ERR_INVALID.
 */
int attn_decode(const void* q, const void* k, const void* v,
                const int32_t* block_table, int max_pages, int page_size, int num_pages,
                const int32_t* seq_lens, int s_max,
                int B, int h, int h_kv, int d_h,
                int chunk_keys, int max_splits, int dtype, float scale,
                float* part_o, float* part_m, float* part_l,
                void* o, float* lse, void* stream);

/*
 * Split-KV decode over 8-bit K/V: K and V hold one OCP E4M3 byte per
 * element (sign, 4 exponent bits with bias 7, 3 mantissa bits; the codes
 * 0x7F and 0xFF are NaN), and each tensor has one fp32 scale: the key and
 * value with codes c stand for e4m3(c) * k_scale and e4m3(c) * v_scale.
 * [OR] section "Where it breaks" (with FP8 K and V the statistics m and l
 * stay fp32); the byte format and the per-tensor scales are this library's
 * choice, the pages fixing none. The products run on the query's 16-bit
 * type (every E4M3 value is exact in fp16 and bf16), the statistics and the
 * partial states in fp32, as attn_decode_split.
 *
 *   q            [B, h, d_h] dtype (ATTN_DTYPE_F16 or ATTN_DTYPE_BF16).
 *   k, v         uint8 codes: contiguous [B, h_kv, s_max, d_h]
 *                (block_table == NULL) or paged pools
 *                [num_pages, page_size, h_kv, d_h]; addressed as in
 *                attn_decode_split with one byte per element.
 *   k_scale, v_scale  finite and > 0 (else ATTN_ERR_INVALID).
 * Everything else (sizes, plans, partial buffers, the written splits,
 * errors) as attn_decode_split; the partials merge with attn_merge_states.
 * Up to 256 query heads per KV head; page sizes any multiple of 16.
 * Groups of 17-128 heads on contiguous K/V, or on pages whose size is a
 * power of two in a pool of under 4 GB, run as the rows of the prefill
 * kernel (as attn_decode_split does for 16-bit K/V); other groups run in
 * blocks of 16 heads. Both forms write the same partial layout.
 */
int attn_decode_split_fp8kv(const void* q, const void* k, const void* v,
                            const int32_t* block_table, int max_pages, int page_size, int num_pages,
                            const int32_t* seq_lens, int s_max,
                            int B, int h, int h_kv, int d_h,
                            int chunk_keys, int max_splits, int dtype, float scale,
                            float k_scale, float v_scale,
                            float* part_o, float* part_m, float* part_l, void* stream);

/*
 * Both decode stages over 8-bit K/V in one call: attn_decode_split_fp8kv
 * into the caller's partial buffers, then attn_merge_states, on `stream`
 * (as attn_decode does for 16-bit K/V).
 *   o            [B, h, d_h] dtype (written); lse [B, h] fp32 or NULL.
 * Errors as attn_decode_split_fp8kv; NULL partials or o: ATTN_ERR_INVALID.
 */
int attn_decode_fp8kv(const void* q, const void* k, const void* v,
                      const int32_t* block_table, int max_pages, int page_size, int num_pages,
                      const int32_t* seq_lens, int s_max,
                      int B, int h, int h_kv, int d_h,
                      int chunk_keys, int max_splits, int dtype, float scale,
                      float k_scale, float v_scale,
                      float* part_o, float* part_m, float* part_l,
                      void* o, float* lse, void* stream);

/*
 * attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops that forbid allocation): the same two
 * stages and results, with the split-KV partial states kept in a scratch
 * array of device memory that the library owns -- 32 MiB, one per GPU,
 * held from the first call on that GPU until the process ends. The call
 * itself allocates nothing. The caller still passes the inputs and o / lse.
 *
 *   Arguments as attn_decode, without part_o / part_m / part_l.
 *   B * h * max_splits * (d_h + 2) * 4 bytes of partial states must fit in
 *   the 32 MiB (e.g. B * h * max_splits <= 64528 for d_h = 128); larger
 *   problems return ATTN_ERR_UNSUPPORTED before anything is launched.
 * Nothing in the scratch needs to start at zero: stage 1 writes every state
 * the merge uses. All calls on one GPU share its scratch: calls that overlap
 * in time on one GPU (different streams, host threads or processes' graphs
 * replayed concurrently) race on it and must be serialised by the caller.
 */
int attn_decode_noalloc(const void* q, const void* k, const void* v,
                        const int32_t* block_table, int max_pages, int page_size, int num_pages,
                        const int32_t* seq_lens, int s_max,
                        int B, int h, int h_kv, int d_h,
                        int chunk_keys, int max_splits, int dtype, float scale,
                        void* o, float* lse, void* stream);

/*
 * Two-operand merge in (O, LSE) form: the output over the union of two
 * disjoint key ranges of the same query rows, from each range's normalised
 * output and LSE (a cascade's shared prefix and per-request suffix, or two
 * context-parallel shards). [NA] sections "The state that gets passed around
 * is the log-sum-exp" (O = w_a O_a + w_b O_b with w = exp(LSE - M) / sum,
 * LSE = M + ln(sum exp(LSE - M)), M the larger LSE) and "Scale first, then
 * multiply" (the weights are normalised before they touch O, so the result
 * is a convex combination); section "The base case is a NaN factory" (an
 * LSE of +inf, the empty-row value of some producers, is read as -inf).
 *
 *   o_a, o_b    [rows, d_h] dtype, normalised outputs of the two ranges.
 *   lse_a, lse_b [rows] fp32 natural-log LSE; -inf or +inf = empty range.
 *   rows        number of (batch, head, query) rows, e.g. B * h * T.
 *   o           [rows, d_h] dtype (written); may alias o_a or o_b.
 *   lse         [rows] fp32 (written) or NULL; may alias lse_a or lse_b.
 * The O of an empty side is never read. Both sides empty: o = +0.0 bits,
 * lse = -inf ([MI], last paragraph).
 */
int attn_merge_lse(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                   int rows, int d_h, void* o, float* lse, int dtype, void* stream);

/*
 * Paged-KV gather: copy each sequence's keys (or values) out of a paged pool
 * into a contiguous tensor, bit for bit. [DA] paged addressing after section
 * "What the merge costs": position p lives in page block_table[b][p / P] at
 * slot p % P.
 *
 *   pool        [num_pages, page_size, h_kv, d_h] dtype
 *   block_table [B, max_pages] int32 device
 *   seq_lens    [B] int32 device, each <= min(s_max, max_pages * page_size)
 *   num_pages   pages in the pool; positions whose page id lies outside
 *               [0, num_pages) are left untouched.
 *   out         [B, h_kv, s_max, d_h] dtype; positions p >= seq_lens[b] are
 *               left untouched. page_size may be any positive value here,
 *               with max_pages * page_size below 2^31 (else
 *               ATTN_ERR_UNSUPPORTED).
 */
int attn_paged_gather(const void* pool, const int32_t* block_table, const int32_t* seq_lens,
                      int B, int h_kv, int d_h, int page_size, int max_pages, int num_pages,
                      int s_max, int dtype, void* out, void* stream);

/*
 * Measurement aid, not part of the attention path: read `bytes` bytes at
 * `src` once, as a plain stream (each of `chunks` workgroups reads one
 * contiguous chunk with 16-byte loads), and write one uint32 per workgroup
 * to out[0 .. chunks) (the xor of the chunk's 32-bit words, so the loads
 * cannot be dropped). Timing it on a kernel's own byte count gives the read
 * rate the device attains at that size -- launch, first-byte latency and
 * drain included -- the floor an HBM-bound kernel such as the split-KV
 * decode is compared with.
 *
 *   src    device pointer, 16-byte aligned; bytes a multiple of 16.
 *   chunks 1 .. 65536 workgroups.
 *   out    [chunks] uint32, device.
 */
int attn_stream_read(const void* src, uint64_t bytes, int chunks, uint32_t* out, void* stream);

/* Message describing the last error returned on the calling thread ("" if
 * none). The pointer stays valid until the next call on that thread. */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

/*
 * Device-side bounds checks (debug build). libattn_checked.so is built from
 * the same sources with ATTN_DEVICE_CHECKS defined: before every global
 * memory access that is not made through a range-checked buffer resource,
 * and for every buffer range a kernel builds, the kernel tests the address
 * against the extent of its tensor, computed from the call's own sizes. A
 * failing access is not made (a load gives zeros, a store is dropped) and
 * the flag of its site (one of ATTN_CHECK_SITES, numbered per kernel and
 * access in the library's sources) is set. Not a page citation: a test aid
 * for the index arithmetic of the kernels above.
 *
 * attn_check_report: after the device is synchronised, copies the flags
 *   (1 = some access at that site failed its test since the last clear) into
 *   hits[0 .. ATTN_CHECK_SITES); n_sites must be at least ATTN_CHECK_SITES.
 * attn_check_clear: sets every flag to 0 (synchronous).
 * attn_check_selftest: launches a kernel on `stream` that tests one address
 *   inside a 64-byte extent from `base` (site 62) and one past it (site 63),
 *   accessing neither: afterwards flag 63 is set and flag 62 is not.
 * In the product library (libattn.so) all three return ATTN_ERR_UNSUPPORTED.
 */
#define ATTN_CHECK_SITES 64
int attn_check_report(uint32_t* hits, int n_sites);
int attn_check_clear(void);
int attn_check_selftest(const void* base, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
