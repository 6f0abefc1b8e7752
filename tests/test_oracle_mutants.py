"""Plant plausible mistakes in copies of the oracle (CPU only) and check that
the pins of tests/test_oracle.py catch each one. A pin set that a wrong
oracle also passes would prove nothing; these tests show that the ones here
fail on: an initial maximum of 0, an accumulator that is not rescaled, the
wrong GQA head mapping, a missing or misplaced scale, top-left causal
alignment, a log-sum-exp in base 2, a merge without the both-empty branch,
a merge that drops the rescale, a gather with the page index and slot
swapped, split slices that drop a key, the wrong GQA head in decode, a merge
that ignores the valid split count, an (O, LSE) merge that averages the two
outputs or reads LSE = +inf as a real mass, and attention that ignores the
key mask."""

import math

import numpy as np
import pytest

import oracle.attention as oatt
import oracle.state as ost
import tests.test_oracle as pins
from tests.conftest import load_golden


def _online_variant(start_ref, rescale_acc):
    """A copy of oracle.state.online_ref with one step changed: the running
    reference starts at ``start_ref``, and the output accumulator is
    multiplied by the decay only if ``rescale_acc``."""
    def online(scores, values, block):
        logits = np.asarray(scores, dtype=np.float64)
        rows = np.asarray(values, dtype=np.float64)
        starts = range(0, logits.size, block)
        refs = np.maximum.accumulate([max(start_ref, float(logits[s:s + block].max())) for s in starts])
        ref, mass, acc = start_ref, 0.0, np.zeros(rows.shape[-1])
        for s, r_new in zip(starts, refs):
            r_new = float(r_new)
            if np.isneginf(r_new):
                continue
            decay = 0.0 if np.isneginf(ref) else math.exp(ref - r_new)
            w = np.exp(logits[s:s + block] - r_new)
            mass = decay * mass + float(w.sum())
            acc = (decay if rescale_acc else 1.0) * acc + w @ rows[s:s + block]
            ref = r_new
        return ref, mass, acc
    return online


# mistake: the running maximum starts at 0 instead of -inf
online_m0 = _online_variant(0.0, True)
# mistake: l is rescaled but the output accumulator is not
online_no_rescale = _online_variant(-np.inf, False)


def _attention_variant(gqa=None, scale_mode="before", causal_mode="bottom_right", log=np.log, use_key_mask=True):
    def att(q, k, v, scale, causal=False, key_mask=None, row_mask=None, rows=None):
        q, k, v = oatt._f64(q), oatt._f64(k), oatt._f64(v)
        b_, h, t_q, d = q.shape
        h_kv, t_k = k.shape[1], k.shape[2]
        g = h // h_kv
        rows = np.arange(t_q) if rows is None else np.asarray(rows)
        o = np.zeros((b_, h, rows.size, v.shape[-1]))
        lse = np.full((b_, h, rows.size), -np.inf)
        for b in range(b_):
            km = None if key_mask is None or not use_key_mask else np.asarray(key_mask)[b]
            rm = None if row_mask is None else np.asarray(row_mask)[b]
            if causal and causal_mode == "top_left":
                vis = oatt.visible_mask(rows, t_k, t_k, True, km, rm)
            else:
                vis = oatt.visible_mask(rows, t_k, t_q, causal, km, rm)
            for i in range(h):
                kv = gqa(i, h, h_kv) if gqa else i // g
                x = q[b, i, rows] @ k[b, kv].T
                if scale_mode == "before":
                    x = scale * x
                x = np.where(vis, x, -np.inf)
                ne = vis.any(axis=1)
                if not ne.any():
                    continue
                xr = x[ne]
                m = xr.max(axis=1)
                p = np.exp(xr - m[:, None])
                l = p.sum(axis=1)
                o[b, i, ne] = (p / l[:, None]) @ v[b, kv]
                lse[b, i, ne] = m + log(l)
        return o, lse
    return att


def _merge_variant(guard_empty, rescale):
    """A copy of the oracle's state fold (oracle.state._combine) for two
    states with one step changed: without the empty-state guard the factors
    are exp(m_i - max) even when every reference is -inf; without the
    rescale every factor is 1."""
    def merge(a, b):
        states = [a, b]
        refs = np.array([float(s[0]) for s in states])
        width = np.asarray(states[0][2], dtype=np.float64).shape[-1]
        live = ~np.isneginf(refs) if guard_empty else np.ones(2, dtype=bool)
        if not live.any():
            return ost.EMPTY_M, 0.0, np.zeros(width)
        top = float(refs[live].max())
        with np.errstate(invalid="ignore"):
            factor = [float(np.exp(r - top)) if rescale else 1.0 for r in refs]
        mass, numer = 0.0, np.zeros(width)
        for f, (_, l_i, a_i) in zip(factor, states):
            mass = mass + l_i * f
            numer = numer + np.asarray(a_i, dtype=np.float64) * f
        return top, mass, numer
    return merge


merge_no_empty_branch = _merge_variant(False, True)
merge_no_rescale = _merge_variant(True, False)


def gather_swapped(pool, block_table, seq_lens, s_max, out=None):
    import torch
    pool_c = pool.detach().cpu()
    bt = np.asarray(block_table)
    n_pages, page, h_kv, d = pool_c.shape
    out = pool_c.new_zeros((bt.shape[0], h_kv, s_max, d)) if out is None else out
    for b in range(bt.shape[0]):
        p = np.arange(int(seq_lens[b]))
        phys = bt[b, p % bt.shape[1]].astype(np.int64)      # mistake: wrong index
        slot = (p // bt.shape[1] % page).astype(np.int64)
        out[b, :, :p.size] = pool_c[torch.from_numpy(phys), torch.from_numpy(slot)].permute(1, 0, 2)
    return out


def split_states_short(q, k, v, seq_len, scale, chunk):
    # mistake: each slice stops one key early
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    h, d = q.shape
    g = h // k.shape[0]
    n = -(-seq_len // chunk) if seq_len > 0 else 0
    m, l, a = np.full((h, n), -np.inf), np.zeros((h, n)), np.zeros((h, n, d))
    for i in range(h):
        x = float(scale) * (k[i // g, :seq_len] @ q[i])
        for s_ in range(n):
            lo, hi = s_ * chunk, min(seq_len, (s_ + 1) * chunk) - 1
            m[i, s_], l[i, s_], a[i, s_] = ost.state_ref(x[lo:hi], v[i // g, lo:hi])
    return m, l, a


def decode_wrong_head(q, k_seqs, v_seqs, seq_lens, scale):
    # mistake: query head i reads KV head i % h_kv instead of i // g
    q = np.asarray(q, dtype=np.float64)
    b_, h, d = q.shape
    o, lse = np.zeros((b_, h, d)), np.full((b_, h), -np.inf)
    for b in range(b_):
        s = int(seq_lens[b])
        kb = np.asarray(k_seqs[b], dtype=np.float64)[:, :s]
        vb = np.asarray(v_seqs[b], dtype=np.float64)[:, :s]
        for i in range(h):
            ob, lb = oatt._rows_attention(q[b, i][None, :], kb[i % kb.shape[0]], vb[i % kb.shape[0]], float(scale),
                                          np.ones((1, s), dtype=bool))
            o[b, i], lse[b, i] = ob[0], lb[0]
    return o, lse


def merge_partials_all(m, l, a, n_valid=None, order=None):
    # mistake: merges every partial row, not only the valid ones
    return ost.merge_partials_ref(m, l, a, n_valid=None, order=order)


def merge_lse_average(o_a, lse_a, o_b, lse_b):
    # mistake: averages the two normalised outputs
    o, lse = ost.merge_lse_ref(o_a, lse_a, o_b, lse_b)
    return 0.5 * (np.asarray(o_a) + np.asarray(o_b)), lse


def merge_lse_inf_as_mass(o_a, lse_a, o_b, lse_b):
    # mistake: an LSE of +inf is taken as a real (infinite) mass
    o_a, o_b = np.asarray(o_a, dtype=np.float64), np.asarray(o_b, dtype=np.float64)
    la, lb = np.asarray(lse_a, dtype=np.float64), np.asarray(lse_b, dtype=np.float64)
    big = np.maximum(la, lb)
    ea, eb = np.exp(la - big), np.exp(lb - big)
    tot = ea + eb
    return o_a * (ea / tot)[..., None] + o_b * (eb / tot)[..., None], big + np.log(tot)


CASES = [
    ("online_ref", online_m0, pins.test_online_row_far_below_zero, ()),
    ("online_ref", online_no_rescale, pins.test_online_equals_safe_softmax_with_late_outlier, (load_golden,)),
    ("attention_ref", _attention_variant(gqa=lambda i, h, hk: i % hk), pins.test_gqa_head_mapping, ()),
    ("attention_ref", _attention_variant(scale_mode="none"), pins.test_causal_row_zero_is_its_single_key, ()),
    ("attention_ref", _attention_variant(scale_mode="none"), pins.test_matches_torch_softmax_and_logsumexp, ()),
    ("attention_ref", _attention_variant(causal_mode="top_left"), pins.test_bottom_right_causal_alignment, ()),
    ("attention_ref", _attention_variant(log=np.log2), pins.test_worked_example_two_blocks, (load_golden,)),
    ("merge_ref", merge_no_empty_branch, pins.test_state_and_merge_empty_branches, ()),
    ("merge_ref", merge_no_rescale, pins.test_worked_example_two_blocks, (load_golden,)),
    ("paged_gather_ref", gather_swapped, pins.test_paged_gather_recovers_ground_truth, ()),
    ("split_states_ref", split_states_short, pins.test_split_partials_merge_to_decode, (32,)),
    ("decode_ref", decode_wrong_head, pins.test_decode_matches_brute_force, ()),
    ("merge_partials_ref", merge_partials_all, pins.test_merge_partials_respects_valid_count, ()),
    ("merge_lse_ref", merge_lse_average, pins.test_merge_lse_two_operand_form, ()),
    ("merge_lse_ref", merge_lse_inf_as_mass, pins.test_merge_lse_two_operand_form, ()),
    ("attention_ref", _attention_variant(use_key_mask=False), pins.test_attention_matches_brute_force,
     (False, True, False, 3, 7)),
]


@pytest.mark.parametrize("name,mutant,pin,args", CASES,
                         ids=[f"{c[0]}-{i}-{c[2].__name__}" for i, c in enumerate(CASES)])
def test_pin_catches_mutant(monkeypatch, name, mutant, pin, args):
    # the unmodified oracle passes the pin ...
    pin(*args)
    # ... and the planted mistake fails it
    monkeypatch.setattr(pins, name, mutant)
    with pytest.raises((AssertionError, FloatingPointError, ValueError)):
        with np.errstate(all="ignore"):
            pin(*args)
