"""Materialised float64 attention: the plain definition the tiled kernels reach.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
``__graft_entry__.smoke()`` and the bench's cpu_baseline leg, never by the
product path.

What is computed, per batch b, query head i and query row t:

1. Logits x_j = scale * <Q[b,i,t,:], K[b,kv(i),j,:]> for every key j, where
   the query head i reads KV head kv(i) = floor(i / g), g = h / h_kv.
   ("Naive attention and the online softmax", opening section: Q is
   [h, T, d_h], K and V are [h_kv, T, d_h] broadcast to the g query heads
   that share them; "Decode attention: FlashDecoding, split-K, paged
   kernels", section "Where GQA enters": row r of a query group belongs to
   query head kv_head * g + r.)
2. A key that is not visible is excluded from the row, not given a large
   negative value ("Merge normalized attention without averaging tile
   outputs", paragraph on fully masked tiles). Visible means: causal
   (j <= t + T_k - T_q, i.e. bottom-right aligned), key mask set, row mask
   set. The scale is applied before the mask ("Naive attention and the
   online softmax", the logits are the row of S after the 1/sqrt(d_h)
   scale and any mask).
3. Safe softmax in three passes: the row maximum m, then the sum
   l = sum_j exp(x_j - m), then the normalised weights exp(x_j - m) / l
   ("Naive attention and the online softmax", section (2) "Safe softmax,
   and why it costs three passes").
4. O = sum_j w_j V[b,kv(i),j,:] and LSE = m + ln l ("Naive attention and the
   online softmax", section "The state that gets passed around is the
   log-sum-exp"; "The Online Softmax Recurrence", section "What it buys").
5. A row with no visible key has no distribution; its output is all zeros
   and its LSE is -inf ("Merge normalized attention without averaging tile
   outputs", last paragraph: zero output is one admissible extension; the
   identity state of the merge is (0, -inf) in "Naive attention and the
   online softmax", section "vLLM: merge_attn_states.cu").

Everything is numpy float64. Inputs are upcast exactly from their stored
fp16/bf16 values; ``scale`` is the float32 value the GPU receives, upcast.
A library matmul serves as the dot-product step; there is no tiling, fusion
or reordering beyond what the definition states.
"""

import numpy as np

# Rows per block when materialising S, to bound memory (2^24 fp64 entries
# = 128 MiB per block). Row blocks do not change the arithmetic: each row is
# computed independently.
_MAX_BLOCK_ELEMS = 1 << 24


def _f64(x):
    """Exact float64 copy of a numpy array or a CPU torch tensor."""
    if hasattr(x, "detach"):  # torch tensor (fp16/bf16/fp32) -> exact upcast
        return x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def visible_mask(t_rows, t_k, t_q, causal, key_mask_row=None, row_mask_row=None):
    """Boolean visibility [len(t_rows), t_k] for one batch entry.

    ``t_rows`` are query indices in [0, t_q). Causal visibility is aligned to
    the bottom-right corner: query t sees key j iff j <= t + t_k - t_q.
    ``key_mask_row`` [t_k] (nonzero = attend) and ``row_mask_row`` [t_q]
    (zero = the whole row is masked) are optional.
    """
    t_rows = np.asarray(t_rows, dtype=np.int64)
    j = np.arange(t_k, dtype=np.int64)
    vis = np.ones((t_rows.size, t_k), dtype=bool)
    if causal:
        vis &= j[None, :] <= (t_rows[:, None] + (t_k - t_q))
    if key_mask_row is not None:
        vis &= (np.asarray(key_mask_row) != 0)[None, :]
    if row_mask_row is not None:
        vis &= (np.asarray(row_mask_row)[t_rows] != 0)[:, None]
    return vis


def _rows_attention(q_rows, k, v, scale, vis):
    """Materialised safe softmax attention for a block of query rows.

    q_rows [R, d], k/v [T_k, d], vis [R, T_k] -> (O [R, d], LSE [R]).
    """
    x = scale * (q_rows @ k.T)                     # logits, scale first
    x = np.where(vis, x, -np.inf)                  # exclusions
    nonempty = vis.any(axis=1)
    o = np.zeros((q_rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.full(q_rows.shape[0], -np.inf, dtype=np.float64)
    if nonempty.any():
        xr = x[nonempty]
        m = xr.max(axis=1)                         # pass 1: row max
        p = np.exp(xr - m[:, None])                # excluded -> exp(-inf) = 0
        l = p.sum(axis=1)                          # pass 2: row sum
        w = p / l[:, None]                         # pass 3: normalise
        o[nonempty] = w @ v
        lse[nonempty] = m + np.log(l)
    return o, lse


def attention_ref(q, k, v, scale, causal=False, key_mask=None, row_mask=None, rows=None):
    """Exact attention in float64 by the plain definition.

    q: [B, h, T_q, d]; k, v: [B, h_kv, T_k, d] (numpy or CPU torch, any float
    dtype; upcast exactly). key_mask: [B, T_k] or None (nonzero = attend).
    row_mask: [B, T_q] or None (zero = the row is fully masked). rows: optional
    1-D array of query indices to evaluate (sampled checks); default all.

    Returns (O [B, h, R, d_v], LSE [B, h, R]) in float64, R = len(rows) or T_q,
    d_v = V's last dimension.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, h, t_q, d = q.shape
    h_kv, t_k = k.shape[1], k.shape[2]
    if h % h_kv:
        raise ValueError("h must be a multiple of h_kv")
    g = h // h_kv
    scale = float(scale)
    rows = np.arange(t_q) if rows is None else np.asarray(rows, dtype=np.int64)
    d_v = v.shape[-1]
    o = np.zeros((b_, h, rows.size, d_v), dtype=np.float64)
    lse = np.full((b_, h, rows.size), -np.inf, dtype=np.float64)
    blk = max(1, _MAX_BLOCK_ELEMS // max(1, t_k))
    for b in range(b_):
        km = None if key_mask is None else np.asarray(key_mask)[b]
        rm = None if row_mask is None else np.asarray(row_mask)[b]
        for r0 in range(0, rows.size, blk):
            rr = rows[r0:r0 + blk]
            vis = visible_mask(rr, t_k, t_q, causal, km, rm)
            for i in range(h):
                kv = i // g
                ob, lb = _rows_attention(q[b, i, rr], k[b, kv], v[b, kv], scale, vis)
                o[b, i, r0:r0 + rr.size] = ob
                lse[b, i, r0:r0 + rr.size] = lb
    return o, lse


def decode_ref(q, k_seqs, v_seqs, seq_lens, scale):
    """One-query-token attention over ragged KV, float64.

    q: [B, h, d]. k_seqs / v_seqs: either padded arrays [B, h_kv, S, d] or a
    list of per-sequence arrays [h_kv, s_b, d]; only keys j < seq_lens[b] are
    attended. The single query sees every one of its s_b keys (the decode
    query is the newest position). A sequence with s_b = 0 gives zeros and
    LSE = -inf.

    Returns (O [B, h, d], LSE [B, h]) float64.
    """
    q = _f64(q)
    b_, h, d = q.shape
    o = np.zeros((b_, h, d), dtype=np.float64)
    lse = np.full((b_, h), -np.inf, dtype=np.float64)
    for b in range(b_):
        s = int(seq_lens[b])
        kb = _f64(k_seqs[b])[:, :s]
        vb = _f64(v_seqs[b])[:, :s]
        h_kv = kb.shape[0]
        g = h // h_kv
        vis = np.ones((1, s), dtype=bool)
        for i in range(h):
            ob, lb = _rows_attention(q[b, i][None, :], kb[i // g], vb[i // g], float(scale), vis)
            o[b, i] = ob[0]
            lse[b, i] = lb[0]
    return o, lse


def paged_gather_ref(pool, block_table, seq_lens, s_max, out=None):
    """Paged-KV gather by plain block-table indexing.

    Position p of sequence b lives in physical page block_table[b, p // P] at
    slot p % P, where P is the page size ("Decode attention: FlashDecoding,
    split-K, paged kernels", the paged addressing after section "What the
    merge costs": the physical block index times the page stride plus the
    in-page offset times the row stride).

    pool: [num_pages, P, h_kv, d] (numpy array of any dtype, or torch).
    block_table: [B, max_pages] int. Returns out [B, h_kv, s_max, d]; positions
    p >= seq_lens[b] keep the values of ``out`` if given, else zeros.
    """
    is_torch = hasattr(pool, "detach")
    pool_c = pool.detach().cpu() if is_torch else np.asarray(pool)
    bt = np.asarray(block_table)
    n_pages, page, h_kv, d = pool_c.shape
    b_ = bt.shape[0]
    if out is None:
        if is_torch:
            out = pool_c.new_zeros((b_, h_kv, s_max, d))
        else:
            out = np.zeros((b_, h_kv, s_max, d), dtype=pool_c.dtype)
    for b in range(b_):
        s = int(seq_lens[b])
        p = np.arange(s)
        phys = bt[b, p // page].astype(np.int64)
        slot = (p % page).astype(np.int64)
        if is_torch:
            import torch  # CPU tensors only; bf16 has no numpy dtype

            rows = pool_c[torch.from_numpy(phys), torch.from_numpy(slot)]   # [s, h_kv, d]
            out[b, :, :s, :] = rows.permute(1, 0, 2)
        else:
            rows = pool_c[phys, slot]                                        # [s, h_kv, d]
            out[b, :, :s, :] = np.transpose(rows, (1, 0, 2))
    return out
