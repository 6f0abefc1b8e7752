"""Seeded synthetic inputs for the attention kernels and their checks.

This module only draws random numbers and lays them out. It holds none of
the attention arithmetic, so both sides of a parity check (the HIP path and
the float64 oracle) may take their inputs from it.

Recipe (the same bytes go to the GPU and, upcast exactly, to the oracle):

* Normal values are drawn with numpy's PCG64 generator as float32
  (``standard_normal``), multiplied by a float32 std when one is given, then
  rounded to the operand dtype by torch (round to nearest even).
* Values are drawn in the order Q, K, V from one stream; integers (lengths,
  page permutation, masks) come from a second stream, so the shapes can be
  known before the values are drawn. Both streams are spawned from
  ``numpy.random.SeedSequence(seed)``.
* Masks are uint8 (1 = attend). A key mask is per batch entry and shared by
  all heads; a row mask marks query rows whose every key is masked.
* Paged KV: each sequence's keys are drawn contiguous, token-major
  ([tokens, h_kv, d]); the token stream of sequence b is cut into pages of
  ``page_size`` tokens and page p of sequence b is stored at physical page
  perm[first_page(b) + p] of the pool [num_pages, page_size, h_kv, d], where
  perm is a seeded random permutation. Slots past the end of a sequence's
  last page, spare pool pages and unused block-table entries (-1) are
  poisoned (NaN for values) so a stray read shows up in the results.

The named workloads are the five shapes the kernels are measured and checked
on (a tiny causal prefill; a Llama-3-8B layer prefill at T=8192; a batch-1
decode at a Llama-3-70B tensor-parallel-8 shard shape over 32768 contiguous
keys; a 64-sequence paged decode at Llama-3-8B shape with ragged lengths;
a prefill numerics stress case with logits of std about 30, tile key masks
and fully masked rows).
"""

import math

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}

# Values are converted to the operand dtype in chunks of this many floats to
# bound host memory for the multi-GB paged pools.
_CHUNK = 1 << 24


def _streams(seed):
    ss = np.random.SeedSequence(int(seed))
    vals, ints = ss.spawn(2)
    return np.random.default_rng(vals), np.random.default_rng(ints)


def _normal(rng, shape, dtype, std=None):
    """Draw N(0, std^2) float32 values in C order and round them to dtype."""
    out = torch.empty(shape, dtype=DTYPES[dtype])
    flat = out.view(-1)
    n = flat.numel()
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(size=hi - lo, dtype=np.float32)
        if std is not None:
            x *= np.float32(std)
        flat[lo:hi] = torch.from_numpy(x).to(out.dtype)
    return out


def default_scale(d):
    """The float32 value of 1/sqrt(d) that the kernels receive."""
    return float(np.float32(1.0 / math.sqrt(d)))


def make_prefill(B, h, h_kv, T_q, T_k, d, dtype, seed, causal=True, qk_std=None,
                 key_tile=64, key_tile_p=0.0, key_p=0.0, row_mask_frac=0.0,
                 row_mask_count=None):
    """Prefill inputs: Q [B,h,T_q,d], K/V [B,h_kv,T_k,d] in ``dtype``.

    qk_std: optional std for Q and K (V stays N(0,1)). key_tile_p: each
    aligned ``key_tile``-key tile of each batch entry is masked with this
    probability. key_p: each single key is masked with this probability.
    row_mask_frac / row_mask_count: that many query rows per batch entry,
    chosen without replacement, have every key masked (row mask 0).
    """
    rv, ri = _streams(seed)
    q = _normal(rv, (B, h, T_q, d), dtype, qk_std)
    k = _normal(rv, (B, h_kv, T_k, d), dtype, qk_std)
    v = _normal(rv, (B, h_kv, T_k, d), dtype)
    key_mask = None
    if key_tile_p > 0.0 or key_p > 0.0:
        key_mask = np.ones((B, T_k), dtype=np.uint8)
        if key_tile_p > 0.0:
            n_tiles = -(-T_k // key_tile)
            dead = ri.random((B, n_tiles)) < key_tile_p
            key_mask &= np.repeat(~dead, key_tile, axis=1)[:, :T_k].astype(np.uint8)
        if key_p > 0.0:
            key_mask &= (ri.random((B, T_k)) >= key_p).astype(np.uint8)
    row_mask = None
    n_rows = row_mask_count
    if n_rows is None and row_mask_frac > 0.0:
        n_rows = int(round(row_mask_frac * T_q))
    if n_rows:
        row_mask = np.ones((B, T_q), dtype=np.uint8)
        for b in range(B):
            row_mask[b, ri.choice(T_q, size=n_rows, replace=False)] = 0
    return dict(kind="prefill", q=q, k=k, v=v, key_mask=key_mask, row_mask=row_mask,
                scale=default_scale(d), causal=bool(causal), dtype=dtype,
                B=B, h=h, h_kv=h_kv, T_q=T_q, T_k=T_k, d=d)


def _e4m3_codes(rng, shape):
    """Random 8-bit E4M3 codes (uint8, OCP layout: sign, 4 exponent bits, 3
    mantissa bits) with the sign and the mantissa uniform and the exponent
    field uniform in 4..9 (magnitudes in [2^-3, 2^3)); never a NaN code.
    One integer in [0, 96) per element, in C order."""
    out = torch.empty(shape, dtype=torch.uint8)
    flat = out.view(-1)
    n = flat.numel()
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        r = rng.integers(0, 96, size=hi - lo, dtype=np.int64)
        codes = ((r // 48) << 7) | ((4 + (r % 48) // 8) << 3) | (r % 8)
        flat[lo:hi] = torch.from_numpy(codes.astype(np.uint8))
    return out


def make_decode(B, h, h_kv, d, dtype, seed, seq_lens=None, len_range=None, paged=False,
                page_size=16, spare_pages=0, poison=True, kv_codes=False):
    """Decode inputs: one query token per sequence, q [B,h,d].

    Lengths: ``seq_lens`` (list) or drawn uniformly from ``len_range``
    (inclusive both ends). Keys/values of sequence b are drawn token-major
    [s_b, h_kv, d] in sequence order (all K first, then all V).

    Contiguous (paged=False): k, v [B, h_kv, S, d] with S = max length;
    positions >= s_b are NaN when ``poison``.
    Paged: k_pool, v_pool [num_pages, page_size, h_kv, d] and block_table
    int32 [B, max_pages] (see the module docstring); num_pages = the pages the
    sequences need + ``spare_pages``.
    Always: k_seqs / v_seqs, per-sequence views [h_kv, s_b, d] of the drawn
    (ground-truth) keys and values.
    kv_codes: K and V are 8-bit E4M3 codes (uint8, see ``_e4m3_codes``)
    instead of ``dtype`` values, and the poison is the NaN code 0x7F.
    """
    rv, ri = _streams(seed)
    if seq_lens is None:
        lo, hi = len_range
        seq_lens = ri.integers(lo, hi, size=B, endpoint=True)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q = _normal(rv, (B, h, d), dtype)
    total = int(seq_lens.sum())
    if kv_codes:
        k_tok = _e4m3_codes(rv, (total, h_kv, d))
        v_tok = _e4m3_codes(rv, (total, h_kv, d))
    else:
        k_tok = _normal(rv, (total, h_kv, d), dtype)
        v_tok = _normal(rv, (total, h_kv, d), dtype)
    kv_dtype = torch.uint8 if kv_codes else DTYPES[dtype]
    offs = np.concatenate([[0], np.cumsum(seq_lens.astype(np.int64))])
    k_seqs = [k_tok[offs[b]:offs[b + 1]].permute(1, 0, 2) for b in range(B)]
    v_seqs = [v_tok[offs[b]:offs[b + 1]].permute(1, 0, 2) for b in range(B)]
    out = dict(kind="decode", q=q, k_seqs=k_seqs, v_seqs=v_seqs, seq_lens=seq_lens,
               scale=default_scale(d), dtype=dtype, B=B, h=h, h_kv=h_kv, d=d,
               paged=bool(paged), kv_codes=bool(kv_codes))
    fill = (0x7F if kv_codes else float("nan")) if poison else 0
    if not paged:
        s_max = int(seq_lens.max()) if B else 0
        k = torch.full((B, h_kv, s_max, d), fill, dtype=kv_dtype)
        v = torch.full((B, h_kv, s_max, d), fill, dtype=kv_dtype)
        for b in range(B):
            k[b, :, :seq_lens[b]] = k_seqs[b]
            v[b, :, :seq_lens[b]] = v_seqs[b]
        out.update(k=k, v=v, s_max=s_max)
        return out
    pages = (seq_lens.astype(np.int64) + page_size - 1) // page_size
    p_used = int(pages.sum())
    n_pages = p_used + int(spare_pages)
    perm = ri.permutation(n_pages)
    max_pages = int(pages.max()) if B else 0
    bt = np.full((B, max(1, max_pages)), -1, dtype=np.int32)
    poffs = np.concatenate([[0], np.cumsum(pages)])
    for b in range(B):
        bt[b, :pages[b]] = perm[poffs[b]:poffs[b + 1]]
    # token t of sequence b -> pool row bt[b, t // page_size] * page_size + t % page_size
    rows = np.empty(total, dtype=np.int64)
    for b in range(B):
        t = np.arange(seq_lens[b], dtype=np.int64)
        rows[offs[b]:offs[b + 1]] = bt[b, t // page_size].astype(np.int64) * page_size + t % page_size
    rows_t = torch.from_numpy(rows)
    k_pool = torch.full((n_pages, page_size, h_kv, d), fill, dtype=kv_dtype)
    v_pool = torch.full((n_pages, page_size, h_kv, d), fill, dtype=kv_dtype)
    k_pool.view(-1, h_kv, d)[rows_t] = k_tok
    v_pool.view(-1, h_kv, d)[rows_t] = v_tok
    out.update(k_pool=k_pool, v_pool=v_pool, block_table=bt, page_size=page_size,
               max_pages=bt.shape[1], num_pages=n_pages)
    return out


def make_chunked_prefill(B, h, h_kv, d, dtype, seed, ctx_range, new_range, page_size=16, spare_pages=0,
                         poison=True):
    """Chunked prefill against a paged cache: sequence b holds T_k,b context
    tokens in the pools (drawn as by ``make_decode`` with ``ctx_range``), the
    last T_q,b of which are new and are the query rows; T_q,b is drawn from
    ``new_range`` (inclusive) and capped at T_k,b. Queries come from a second
    pair of streams (root seed ``seed + 7919``) and are packed token-major.

    Returns the paged decode dict plus q [total_q, h, d], cu_seqlens_q
    int32 [B+1], q_lens int32 [B] and seq_lens_k (= seq_lens).
    """
    dec = make_decode(B, h, h_kv, d, dtype, seed, len_range=ctx_range, paged=True, page_size=page_size,
                      spare_pages=spare_pages, poison=poison)
    rv, ri = _streams(seed + 7919)
    lo, hi = new_range
    q_lens = np.minimum(ri.integers(lo, hi, size=B, endpoint=True), dec["seq_lens"]).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(q_lens.astype(np.int64))]).astype(np.int32)
    q = _normal(rv, (int(cu[-1]), h, d), dtype)
    dec.update(kind="chunked_prefill", q=q, q_lens=q_lens, cu_seqlens_q=cu, seq_lens_k=dec["seq_lens"],
               max_q=int(q_lens.max()) if B else 0)
    return dec


# The named workloads. Seeds are 1000 + their position (1-based); the sixth
# is the chunked-prefill shape of the paged prefill entry point.
CONFIGS = {
    "tiny_prefill": dict(
        kind="prefill", B=1, h=4, h_kv=1, T_q=256, T_k=256, d=128, dtype="f16",
        causal=True, seed=1001),
    "llama3_8b_prefill_t8192": dict(
        kind="prefill", B=1, h=32, h_kv=8, T_q=8192, T_k=8192, d=128, dtype="bf16",
        causal=True, seed=1002),
    "decode_70b_tp8_s32768": dict(
        kind="decode", B=1, h=8, h_kv=1, d=128, dtype="bf16", seq_lens=[32768],
        paged=False, seed=1003),
    "paged_decode_llama3_8b_b64": dict(
        kind="decode", B=64, h=32, h_kv=8, d=128, dtype="bf16", len_range=(512, 16384),
        paged=True, page_size=16, seed=1004),
    "stress_prefill_t4096": dict(
        kind="prefill", B=1, h=32, h_kv=8, T_q=4096, T_k=4096, d=128, dtype="bf16",
        causal=True, qk_std=math.sqrt(30.0), key_tile=64, key_tile_p=1.0 / 8.0,
        row_mask_frac=0.01, seed=1005),
    "chunked_prefill_llama3_8b_b8": dict(
        kind="chunked_prefill", B=8, h=32, h_kv=8, d=128, dtype="bf16", ctx_range=(1024, 8192),
        new_range=(256, 1024), page_size=16, seed=1006),
}


def make_config(name, **overrides):
    """Build the named workload (optionally with some fields overridden)."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    if kind == "prefill":
        return make_prefill(**cfg)
    if kind == "chunked_prefill":
        return make_chunked_prefill(**cfg)
    return make_decode(**cfg)
