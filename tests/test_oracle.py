"""Pins for the float64 oracle (CPU only).

Each test ties an oracle function to something other than itself: a value
the pages print (fixtures under tests/golden/, each with its citation), a
closed form, an invariant, a library routine on a special case, or brute
force on tiny inputs. tests/test_oracle_mutants.py plants plausible mistakes
in copies of the oracle and shows that these pins catch them.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (
    attention_ref,
    brute_attention,
    decode_ref,
    finalize_ref,
    merge_lse_ref,
    merge_partials_ref,
    merge_ref,
    online_ref,
    paged_gather_ref,
    split_states_ref,
    state_ref,
)
from online_softmax_tiled_amd.workloads import make_decode, make_prefill


def rounded(x, decimals):
    return float(np.round(x, decimals))


def softmax_row_ref(x, v):
    """Materialised attention on a bare logit row through the oracle: d = 1,
    q = 1, k = x, scale = 1 makes the logits exactly x."""
    x = np.asarray(x, dtype=np.float64)
    vis = ~np.isneginf(x)
    kk = np.where(vis, x, 0.0)
    q = np.ones((1, 1, 1, 1))
    k = kk.reshape(1, 1, -1, 1)
    vv = np.asarray(v, dtype=np.float64).reshape(1, 1, x.size, -1)
    o, lse = attention_ref(q, k, vv, 1.0, key_mask=vis.reshape(1, -1).astype(np.uint8))
    return o[0, 0, 0], lse[0, 0, 0]


# ---------------------------------------------------------------- worked examples

def test_worked_example_two_blocks(golden):
    g = golden("worked_example_two_blocks.json")
    dec = g["printed_decimals"]
    b1, b2 = (np.array(b) for b in g["blocks"])
    v1 = np.zeros((2, 1))
    st1 = state_ref(b1, v1)
    assert st1[0] == g["after_block_1"]["m"]
    assert rounded(st1[1], dec) == g["after_block_1"]["l"]
    # the streaming recurrence over the whole row
    m, l, _ = online_ref(np.concatenate([b1, b2]), np.zeros((4, 1)), block=2)
    assert m == g["after_block_2"]["m"]
    assert rounded(l, dec) == g["after_block_2"]["l"]
    resc = math.exp(st1[0] - m)
    assert rounded(resc, dec) == g["after_block_2"]["rescale"]
    assert rounded(st1[1] * resc, dec) == g["after_block_2"]["old_l_rescaled"]
    # the symmetric merge gives the same state
    mm, lm, _ = merge_ref(st1, state_ref(b2, np.zeros((2, 1))))
    assert mm == m and abs(lm - l) < 1e-15
    # exact closed form: the direct sum relative to the true max
    exact = 1.0 + math.exp(-2) + math.exp(-3) + math.exp(-4)
    assert rounded(exact, dec) == g["direct_sum"]
    assert abs(l - exact) < 1e-15
    # LSE of the row by the materialised oracle
    _, lse = softmax_row_ref([3.0, 1.0, 5.0, 2.0], np.zeros((4, 1)))
    assert abs(lse - (5.0 + math.log(exact))) < 1e-14


def test_verify_on_numbers_rescale(golden):
    g = golden("verify_on_numbers_rescale.json")
    x = np.array(g["logits_ours"])
    blk = g["block"]
    rng = np.random.default_rng(7)
    v = rng.normal(size=(x.size, 5))
    st2 = online_ref(x[:2 * blk], v[:2 * blk], blk)
    assert st2[0] == g["max_before_block_3"]
    st3 = online_ref(x[:3 * blk], v[:3 * blk], blk)
    assert st3[0] == g["max_after_block_3"]
    alpha = math.exp(st2[0] - st3[0])
    assert float(f"{alpha:.{g['rescale_sig_digits'] - 1}e}") == g["rescale_printed"]
    assert round(1.0 / alpha) == g["divisor_printed"]
    # the third step is exactly alpha-rescaled old state plus the new block
    p3 = np.exp(x[2 * blk:3 * blk] - st3[0])
    assert abs(st3[1] - (alpha * st2[1] + p3.sum())) < 1e-15
    np.testing.assert_allclose(st3[2], alpha * st2[2] + p3 @ v[2 * blk:3 * blk], rtol=1e-15, atol=1e-15)
    # and the final state equals the direct computation
    o, lse = finalize_ref(online_ref(x, v, blk))
    o_ref, lse_ref = softmax_row_ref(x, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-14, atol=1e-14)
    assert abs(lse - lse_ref) < 1e-14


def test_online_equals_safe_softmax_with_late_outlier(golden):
    g = golden("online_vs_safe_softmax_check.json")
    rng = np.random.default_rng(0)
    x = rng.normal(0, g["logit_std"], g["keys"])
    x[g["outlier_index"]] = g["outlier_value"]
    v = rng.normal(0, 1, (g["keys"], g["head_dim"]))
    o, lse = finalize_ref(online_ref(x, v, g["block"]))
    o_ref, lse_ref = softmax_row_ref(x, v)
    np.testing.assert_allclose(o, o_ref, rtol=g["rtol"], atol=g["atol"])
    assert abs(lse - lse_ref) <= g["atol"] + g["rtol"] * abs(lse_ref)
    assert lse_ref >= g["outlier_value"]  # the outlier dominates the row


def _uneven_blocks(rng, n):
    cuts = sorted(rng.choice(np.arange(2, n - 1), size=9, replace=False).tolist())
    edges = [0, 1] + cuts + [n]          # first block has length 1
    return [(edges[i], edges[i + 1]) for i in range(len(edges) - 1) if edges[i + 1] > edges[i]]


def test_merge_order_invariance(golden):
    g = golden("merge_order_invariance.json")
    rng = np.random.default_rng(11)
    n = g["keys"]
    x = rng.normal(0, g["score_std"], n)
    v = rng.normal(0, 1, (n, 16))
    blocks = _uneven_blocks(rng, n)
    assert blocks[0][1] - blocks[0][0] == 1
    masked = 3                            # one block fully masked
    x[blocks[masked][0]:blocks[masked][1]] = -np.inf
    states = [state_ref(x[a:b], v[a:b]) for a, b in blocks]
    assert np.isneginf(states[masked][0]) and states[masked][1] == 0.0
    m = np.array([s[0] for s in states])
    l = np.array([s[1] for s in states])
    a = np.stack([s[2] for s in states])
    k = len(states)
    orders = {
        "sequential": list(range(k)),
        "reversed": list(range(k))[::-1],
        "shuffled": rng.permutation(k).tolist(),
        "tree": (((0, 1), (2, 3)), ((4, 5), (6, (7, 8))), (9, 10)),
    }
    o_ref, lse_ref = softmax_row_ref(x, v)
    outs = {name: merge_partials_ref(m, l, a, order=o) for name, o in orders.items()}
    outs["one_shot"] = merge_partials_ref(m, l, a)
    for name, (o, lse) in outs.items():
        err = np.max(np.abs(o - o_ref)) / np.max(np.abs(o_ref))
        assert err < 1e-13, (name, err)
        assert abs(lse - lse_ref) / abs(lse_ref) < 1e-14, name


# ------------------------------------------------------------------ brute force

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("use_key_mask", [False, True])
@pytest.mark.parametrize("use_row_mask", [False, True])
@pytest.mark.parametrize("t_q,t_k", [(1, 5), (3, 7), (5, 5), (6, 4)])
def test_attention_matches_brute_force(causal, use_key_mask, use_row_mask, t_q, t_k):
    rng = np.random.default_rng(hash((causal, use_key_mask, use_row_mask, t_q, t_k)) % 2**32)
    B, h, h_kv, d = 2, 4, 2, 3
    q = rng.normal(size=(B, h, t_q, d))
    k = rng.normal(size=(B, h_kv, t_k, d)) * 2.0
    v = rng.normal(size=(B, h_kv, t_k, d))
    km = (rng.random((B, t_k)) < 0.6).astype(np.uint8) if use_key_mask else None
    if km is not None:
        km[1, :] = 0                      # batch 1: every key masked
    rm = (rng.random((B, t_q)) < 0.7).astype(np.uint8) if use_row_mask else None
    scale = 0.7
    o, lse = attention_ref(q, k, v, scale, causal, km, rm)
    ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal,
                             None if km is None else km.tolist(),
                             None if rm is None else rm.tolist())
    ob, lb = np.array(ob), np.array(lb)
    np.testing.assert_allclose(o, ob, rtol=1e-13, atol=1e-14)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-13, atol=1e-14)
    if use_key_mask:
        assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))


def test_decode_matches_brute_force():
    rng = np.random.default_rng(3)
    B, h, h_kv, d = 3, 6, 2, 4
    lens = [0, 1, 9]
    q = rng.normal(size=(B, h, d))
    ks = [rng.normal(size=(h_kv, s, d)) for s in lens]
    vs = [rng.normal(size=(h_kv, s, d)) for s in lens]
    o, lse = decode_ref(q, ks, vs, lens, 0.5)
    for b, s in enumerate(lens):
        if s == 0:
            assert np.all(o[b] == 0.0) and np.all(np.isneginf(lse[b]))
            continue
        ob, lb = brute_attention(q[b][None, :, None, :].tolist(), ks[b][None].tolist(),
                                 vs[b][None].tolist(), 0.5)
        np.testing.assert_allclose(o[b], np.array(ob)[0, :, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[b], np.array(lb)[0, :, 0], rtol=1e-13)


# ------------------------------------------------------------------ closed forms

def _rand_case(seed, B=1, h=4, h_kv=2, t=33, d=8):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(B, h, t, d)), rng.normal(size=(B, h_kv, t, d)),
            rng.normal(size=(B, h_kv, t, d)), rng)


def test_causal_row_zero_is_its_single_key():
    q, k, v, _ = _rand_case(1)
    o, lse = attention_ref(q, k, v, 0.3, causal=True)
    g = 2
    for i in range(4):
        assert np.array_equal(o[0, i, 0], v[0, i // g, 0])           # exactly v_0
        assert lse[0, i, 0] == 0.3 * float(q[0, i, 0] @ k[0, i // g, 0])


def test_zero_query_gives_mean_and_log_count():
    q, k, v, _ = _rand_case(2)
    q[:] = 0.0
    o, lse = attention_ref(q, k, v, 0.3, causal=True)
    for t in range(q.shape[2]):
        for i in range(4):
            np.testing.assert_allclose(o[0, i, t], v[0, i // 2, :t + 1].mean(axis=0), rtol=1e-13, atol=1e-15)
            assert abs(lse[0, i, t] - math.log(t + 1)) < 1e-14


def test_constant_values_pass_through():
    q, k, v, _ = _rand_case(3)
    v[:] = 1.75
    o, _ = attention_ref(q, k * 5, v, 1.0, causal=True)
    np.testing.assert_allclose(o, 1.75, rtol=1e-14)


def test_gqa_head_mapping():
    # query head i reads KV head i // g: with values equal to the KV head
    # index, every output equals that index.
    B, h, h_kv, t, d = 1, 8, 2, 9, 4
    rng = np.random.default_rng(4)
    q = rng.normal(size=(B, h, t, d))
    k = rng.normal(size=(B, h_kv, t, d))
    v = np.zeros((B, h_kv, t, d))
    v[0, 1] = 1.0
    o, _ = attention_ref(q, k, v, 0.5, causal=False)
    for i in range(h):
        np.testing.assert_allclose(o[0, i], np.full((t, d), float(i // (h // h_kv))), rtol=1e-14, atol=1e-14)
    # and the keys of head i's group decide its weights: the decode oracle agrees
    od, _ = decode_ref(q[:, :, -1], [k[0]], [v[0]], [t], 0.5)
    np.testing.assert_allclose(od[0], o[0, :, -1], rtol=1e-14)


def test_fully_masked_rows_are_zero_and_neg_inf():
    q, k, v, _ = _rand_case(5)
    km = np.zeros((1, q.shape[2]), dtype=np.uint8)
    o, lse = attention_ref(q, k, v, 0.3, causal=True, key_mask=km)
    assert np.all(o == 0.0) and not np.any(np.signbit(o)) and np.all(np.isneginf(lse))
    rm = np.ones((1, q.shape[2]), dtype=np.uint8)
    rm[0, [0, 7, 32]] = 0
    o, lse = attention_ref(q, k, v, 0.3, causal=True, row_mask=rm)
    for t in (0, 7, 32):
        assert np.all(o[0, :, t] == 0.0) and np.all(np.isneginf(lse[0, :, t]))
    assert np.all(np.isfinite(lse[0, :, 1]))


def test_convexity_and_lse_bounds():
    q, k, v, rng = _rand_case(6, t=40)
    km = (rng.random((1, 40)) < 0.5).astype(np.uint8)
    km[0, 0] = 1
    scale = 2.0
    o, lse = attention_ref(q, k, v, scale, causal=True, key_mask=km)
    for i in range(4):
        for t in range(40):
            vis = [j for j in range(t + 1) if km[0, j]]
            vv = v[0, i // 2, vis]
            assert np.all(o[0, i, t] >= vv.min(axis=0) - 1e-13)
            assert np.all(o[0, i, t] <= vv.max(axis=0) + 1e-13)
            x = scale * (k[0, i // 2, vis] @ q[0, i, t])
            assert x.max() - 1e-12 <= lse[0, i, t] <= x.max() + math.log(len(vis)) + 1e-12


def test_matches_torch_softmax_and_logsumexp():
    # textbook special case: the library's softmax/logsumexp in float64
    q, k, v, rng = _rand_case(8, h=4, h_kv=1, t=50, d=16)
    o, lse = attention_ref(q, k * 3, v, 0.25, causal=True)
    qt, kt, vt = (torch.from_numpy(a) for a in (q, k * 3, v))
    x = 0.25 * (qt[0] @ kt[0, 0].T)                         # [h, t, t]
    causal = torch.ones(50, 50, dtype=torch.bool).tril()
    x = x.masked_fill(~causal, float("-inf"))
    w = torch.softmax(x, dim=-1)
    np.testing.assert_allclose(o[0], (w @ vt[0, 0]).numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], torch.logsumexp(x, dim=-1).numpy(), rtol=1e-13)


def test_bottom_right_causal_alignment():
    # T_q < T_k: the last query row sees every key, the first sees T_k - T_q + 1
    q, k, v, _ = _rand_case(9, t=12)
    q = q[:, :, :4]
    o, _ = attention_ref(q, k, v, 0.5, causal=True)
    o_full, _ = attention_ref(q, k, v, 0.5, causal=False)
    np.testing.assert_allclose(o[0, :, -1], o_full[0, :, -1], rtol=1e-14)
    o_first, _ = attention_ref(q[:, :, :1], k[:, :, :9], v[:, :, :9], 0.5, causal=False)
    np.testing.assert_allclose(o[0, :, 0], o_first[0, :, 0], rtol=1e-14)


def test_large_logits_do_not_overflow():
    # logits far beyond exp's float64 range are fine after the max shift
    q, k, v, _ = _rand_case(10)
    o, lse = attention_ref(q * 40, k * 40, v, 1.0, causal=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert lse.max() > 710.0            # exp(lse) would overflow float64


def test_sampled_rows_equal_full():
    q, k, v, rng = _rand_case(12, t=30)
    km = (rng.random((1, 30)) < 0.8).astype(np.uint8)
    rows = np.array([29, 0, 13])
    o, lse = attention_ref(q, k, v, 0.5, True, km, rows=rows)
    of, lf = attention_ref(q, k, v, 0.5, True, km)
    np.testing.assert_array_equal(o, of[:, :, rows])
    np.testing.assert_array_equal(lse, lf[:, :, rows])


# ------------------------------------------------------------- states and merges

def test_state_and_merge_empty_branches():
    d = 3
    empty = state_ref(np.array([]), np.zeros((0, d)))
    assert np.isneginf(empty[0]) and empty[1] == 0.0 and np.all(empty[2] == 0.0)
    empty2 = state_ref(np.array([-np.inf, -np.inf]), np.full((2, d), np.nan))
    assert np.isneginf(empty2[0]) and empty2[1] == 0.0
    a = state_ref(np.array([0.5, -1.0]), np.arange(6.0).reshape(2, 3))
    with np.errstate(invalid="raise"):
        mm = merge_ref(a, empty)
        assert mm[0] == a[0] and mm[1] == a[1] and np.array_equal(mm[2], a[2])     # identity
        mm = merge_ref(empty, a)
        assert mm[0] == a[0] and mm[1] == a[1] and np.array_equal(mm[2], a[2])
        ee = merge_ref(empty, empty2)
        assert np.isneginf(ee[0]) and ee[1] == 0.0 and not np.any(np.isnan(ee[2]))
    o, lse = finalize_ref(ee)
    assert np.all(o == 0.0) and np.isneginf(lse)


def test_merge_commutes_and_associates():
    rng = np.random.default_rng(13)
    x = rng.normal(0, 10, 30)
    v = rng.normal(size=(30, 4))
    s = [state_ref(x[i:i + 10], v[i:i + 10]) for i in (0, 10, 20)]
    ab = merge_ref(s[0], s[1])
    ba = merge_ref(s[1], s[0])
    assert ab[0] == ba[0] and abs(ab[1] - ba[1]) < 1e-15
    left = finalize_ref(merge_ref(merge_ref(s[0], s[1]), s[2]))
    right = finalize_ref(merge_ref(s[0], merge_ref(s[1], s[2])))
    np.testing.assert_allclose(left[0], right[0], rtol=1e-14)
    whole = finalize_ref(state_ref(x, v))
    np.testing.assert_allclose(left[0], whole[0], rtol=1e-13)
    assert abs(left[1] - whole[1]) < 1e-13


@pytest.mark.parametrize("chunk", [1, 16, 100, 128, 1000])
def test_split_partials_merge_to_decode(chunk):
    rng = np.random.default_rng(chunk)
    h, h_kv, d, s = 8, 2, 16, 300
    q = rng.normal(size=(h, d))
    k = rng.normal(size=(h_kv, s, d)) * 3
    v = rng.normal(size=(h_kv, s, d))
    m, l, a = split_states_ref(q, k, v, s, 0.3, chunk)
    assert m.shape[1] == -(-s // chunk)
    o_ref, lse_ref = decode_ref(q[None], [k], [v], [s], 0.3)
    for i in range(h):
        o, lse = merge_partials_ref(m[i], l[i], a[i])
        np.testing.assert_allclose(o, o_ref[0, i], rtol=1e-12, atol=1e-14)
        assert abs(lse - lse_ref[0, i]) < 1e-12
        # a partial finalised alone is attention over its own key slice
        o0, lse0 = finalize_ref((m[i, 0], l[i, 0], a[i, 0]))
        hi = min(s, chunk)
        o_s, lse_s = decode_ref(q[None], [k[:, :hi]], [v[:, :hi]], [hi], 0.3)
        np.testing.assert_allclose(o0, o_s[0, i], rtol=1e-12, atol=1e-14)
        assert abs(lse0 - lse_s[0, i]) < 1e-12


def test_merge_partials_respects_valid_count():
    rng = np.random.default_rng(14)
    m = rng.normal(size=6)
    l = rng.random(6) + 0.5
    a = rng.normal(size=(6, 3))
    m_poison = m.copy()
    m_poison[4:] = np.nan
    o1, lse1 = merge_partials_ref(m, l, a, n_valid=4)
    o2, lse2 = merge_partials_ref(m_poison, l, a, n_valid=4)
    np.testing.assert_array_equal(o1, o2)
    assert lse1 == lse2
    o0, lse0 = merge_partials_ref(m, l, a, n_valid=0)
    assert np.all(o0 == 0.0) and np.isneginf(lse0)


def test_merge_lse_two_operand_form():
    q, k, v, rng = _rand_case(15, t=24)
    km_a = np.zeros((1, 24), dtype=np.uint8)
    km_a[0, :10] = 1
    km_b = 1 - km_a
    oa, la = attention_ref(q, k, v, 0.5, key_mask=km_a)
    ob, lb = attention_ref(q, k, v, 0.5, key_mask=km_b)
    of, lf = attention_ref(q, k, v, 0.5)
    o, lse = merge_lse_ref(oa, la, ob, lb)
    np.testing.assert_allclose(o, of, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, lf, rtol=1e-14)
    o2, _ = merge_lse_ref(ob, lb, oa, la)
    np.testing.assert_allclose(o2, o, rtol=1e-15, atol=1e-16)
    # empty sides: -inf and +inf both read as empty; both empty -> zeros, -inf
    z = np.zeros_like(oa)
    ninf = np.full_like(la, -np.inf)
    pinf = np.full_like(la, np.inf)
    with np.errstate(invalid="raise"):
        o3, l3 = merge_lse_ref(oa, la, z, ninf)
        np.testing.assert_array_equal(o3, oa)
        np.testing.assert_allclose(l3, la, rtol=0, atol=0)
        o4, l4 = merge_lse_ref(z, pinf, oa, la)
        np.testing.assert_array_equal(o4, oa)
        o5, l5 = merge_lse_ref(z, pinf, z, ninf)
    assert np.all(o5 == 0.0) and np.all(np.isneginf(l5))
    # scale-first keeps huge masses finite: a convex combination
    big = np.full_like(la, 1e4)
    o6, l6 = merge_lse_ref(oa, big, ob, big - 1.0)
    assert np.all(np.isfinite(o6)) and np.all(np.abs(o6) <= np.maximum(np.abs(oa), np.abs(ob)) + 1e-12)


# ------------------------------------------------------------------ paged gather

def test_paged_gather_recovers_ground_truth():
    dec = make_decode(B=5, h=4, h_kv=2, d=8, dtype="bf16", seed=77, len_range=(1, 70),
                      paged=True, page_size=16, spare_pages=3)
    s_max = int(dec["seq_lens"].max())
    sentinel = torch.full((5, 2, s_max, 8), 123.0, dtype=torch.bfloat16)
    out = paged_gather_ref(dec["k_pool"], dec["block_table"], dec["seq_lens"], s_max, out=sentinel.clone())
    for b in range(5):
        s = int(dec["seq_lens"][b])
        assert torch.equal(out[b, :, :s], dec["k_seqs"][b])
        assert torch.all(out[b, :, s:] == 123.0)
    # numpy path, with a page size larger than 16
    dec2 = make_decode(B=3, h=2, h_kv=1, d=4, dtype="f16", seed=78, len_range=(1, 100),
                       paged=True, page_size=32)
    pool_np = dec2["v_pool"].numpy()
    out2 = paged_gather_ref(pool_np, dec2["block_table"], dec2["seq_lens"], int(dec2["seq_lens"].max()))
    for b in range(3):
        s = int(dec2["seq_lens"][b])
        np.testing.assert_array_equal(out2[b, :, :s], dec2["v_seqs"][b].numpy())


def test_paged_pool_poison_and_table():
    dec = make_decode(B=4, h=4, h_kv=2, d=8, dtype="bf16", seed=79, len_range=(1, 40),
                      paged=True, spare_pages=2)
    bt, lens = dec["block_table"], dec["seq_lens"]
    used = set()
    for b in range(4):
        n = -(-int(lens[b]) // 16)
        assert np.all(bt[b, :n] >= 0) and np.all(bt[b, n:] == -1)
        used.update(bt[b, :n].tolist())
        last = int(bt[b, n - 1])
        tail = int(lens[b]) - (n - 1) * 16
        assert torch.all(torch.isnan(dec["k_pool"][last, tail:].float()))
    assert len(used) == dec["num_pages"] - 2
    spare = sorted(set(range(dec["num_pages"])) - used)
    assert torch.all(torch.isnan(dec["v_pool"][spare].float()))


# ---------------------------------------------------------- the named workloads

def test_named_workload_shapes_and_determinism():
    from online_softmax_tiled_amd.workloads import make_config
    c1 = make_config("tiny_prefill")
    assert c1["q"].shape == (1, 4, 256, 128) and c1["k"].shape == (1, 1, 256, 128)
    assert c1["q"].dtype == torch.float16 and c1["causal"]
    assert c1["scale"] == float(np.float32(1 / math.sqrt(128)))
    again = make_config("tiny_prefill")
    assert torch.equal(c1["q"], again["q"]) and torch.equal(c1["v"], again["v"])
    c5 = make_config("stress_prefill_t4096", T_q=512, T_k=512)
    assert c5["row_mask"].sum() == 512 - round(0.01 * 512)
    km = c5["key_mask"][0].reshape(-1, 64)
    assert np.all((km.min(axis=1) == km.max(axis=1)))      # whole aligned tiles
    # logit std ~ 30 for the stress case
    x = c5["scale"] * (c5["q"][0, 0].double() @ c5["k"][0, 0].double().T)
    assert 25.0 < float(x.std()) < 35.0


def test_online_row_far_below_zero():
    # softmax is shift invariant: a row of logits near -1000 must give the
    # same result as the same row shifted to near 0 (an initial maximum of 0
    # instead of -inf would underflow every term here).
    rng = np.random.default_rng(16)
    x = rng.normal(size=200)
    v = rng.normal(size=(200, 8))
    o, lse = finalize_ref(online_ref(x - 1000.0, v, 64))
    o0, lse0 = softmax_row_ref(x, v)
    np.testing.assert_allclose(o, o0, rtol=1e-12, atol=1e-14)
    assert abs(lse - (lse0 - 1000.0)) < 1e-9
