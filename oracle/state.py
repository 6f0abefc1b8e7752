"""Partial softmax states and their merges, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A state summarises a set of keys for one query row as (m, l, a):
m is the largest logit of the set, l = sum exp(x - m) and
a = sum exp(x - m) v, a d-vector ("The Online Softmax Recurrence", section
"The recurrence"). The empty set is (-inf, 0, 0) ("Naive attention and the
online softmax", section "The proof": the maximum of the empty set is -inf
and its sum is 0; "Merge normalized attention without averaging tile
outputs", paragraph on fully masked tiles: an empty summary with zero mass
and zero numerator).

These functions are used to check merge arithmetic and the GPU's split-KV
partials. The reference *outputs* of attention come from
:func:`oracle.attention.attention_ref`, the materialised definition.
"""

import math

import numpy as np

EMPTY_M = -np.inf


def state_ref(scores, values):
    """Partial state (m, l, a) of one block of keys.

    scores: [n] logits of the block (-inf marks an excluded key); values:
    [n, d]. A block with no keys, or with every key excluded, is the empty
    state (-inf, 0, zeros) -- returned by an explicit branch so that
    -inf - (-inf) is never formed ("The Online Softmax Recurrence", section
    "Worked example", the state function's empty-block branch, and section
    "Where it breaks").
    """
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    d = values.shape[-1]
    if scores.size == 0 or np.all(np.isneginf(scores)):
        return EMPTY_M, 0.0, np.zeros(d)
    m = float(scores.max())
    p = np.exp(scores - m)
    return m, float(p.sum()), p @ values


def merge_ref(a, b):
    """Merge two states of disjoint key sets.

    The new reference is the larger maximum; each side's mass and numerator
    are multiplied by exp(old max - new max), a factor in [0, 1], then added
    ("Merge normalized attention without averaging tile outputs", paragraph
    on disjoint nonempty tiles; "The Online Softmax Recurrence", section
    "The recurrence", the general two-state form). If both sides are empty
    the result is the empty state, by an explicit branch
    ("Merge normalized attention without averaging tile outputs", paragraph
    on fully masked tiles). An empty side has m = -inf and contributes
    exp(-inf) = 0 against a finite maximum.
    """
    (ma, la, xa), (mb, lb, xb) = a, b
    m = max(ma, mb)
    if np.isneginf(m):
        return EMPTY_M, 0.0, np.zeros_like(np.asarray(xa, dtype=np.float64))
    sa = math.exp(ma - m) if not np.isneginf(ma) else 0.0
    sb = math.exp(mb - m) if not np.isneginf(mb) else 0.0
    return m, la * sa + lb * sb, np.asarray(xa) * sa + np.asarray(xb) * sb


def finalize_ref(state):
    """(m, l, a) -> (O, LSE) = (a / l, m + ln l); the empty state gives
    (zeros, -inf) ("The Online Softmax Recurrence", sections "The recurrence"
    and "What it buys": o = a / l and the log-sum-exp m + ln l; zero output
    for a row with no keys, "Merge normalized attention without averaging
    tile outputs", last paragraph)."""
    m, l, a = state
    a = np.asarray(a, dtype=np.float64)
    if l == 0.0:
        return np.zeros_like(a), -np.inf
    return a / l, m + math.log(l)


def online_ref(scores, values, block):
    """One left-to-right pass over the row in blocks of ``block`` keys.

    The streaming recurrence of "Naive attention and the online softmax",
    section (3) "The online recurrence", extended to the output in section
    "Extending the recurrence to the output": with the running state
    (m, l, O~) starting at (-inf, 0, 0), each block B raises the maximum to
    m' = max(m, max B), forms alpha = exp(m - m'), and sets
    l <- alpha l + sum_B exp(x - m'), O~ <- alpha O~ + sum_B exp(x - m') v.
    alpha is taken as 0 while the old maximum is still -inf (the base-case
    guard of that page's numerical check), and a block that leaves the
    maximum at -inf (nothing visible yet) leaves the state unchanged.

    Returns the final state (m, l, O~); divide once at the end with
    :func:`finalize_ref`.
    """
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    m, l, o = EMPTY_M, 0.0, np.zeros(values.shape[-1])
    for j in range(0, scores.size, block):
        xb, vb = scores[j:j + block], values[j:j + block]
        m_new = max(m, float(xb.max())) if xb.size else m
        if np.isneginf(m_new):
            continue                              # still empty: no -inf - -inf
        alpha = math.exp(m - m_new) if not np.isneginf(m) else 0.0
        p = np.exp(xb - m_new)
        l = alpha * l + float(p.sum())
        o = alpha * o + p @ vb
        m = m_new
    return m, l, o


def split_states_ref(q, k, v, seq_len, scale, chunk):
    """Split-KV partial states for one sequence and one query token.

    q: [h, d]; k, v: [h_kv, >= seq_len, d]. The keys [0, seq_len) are cut into
    contiguous slices of ``chunk`` keys, the last one possibly shorter
    ("Decode attention: FlashDecoding, split-K, paged kernels", opening
    section and section "Segment length, and the early exit"). Each slice
    yields the state of its keys for every query head (query head i reads KV
    head i // g).

    Returns (m [h, S], l [h, S], a [h, S, d]) with S = ceil(seq_len / chunk).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    h, d = q.shape
    g = h // k.shape[0]
    n_split = -(-seq_len // chunk) if seq_len > 0 else 0
    m = np.full((h, n_split), -np.inf)
    l = np.zeros((h, n_split))
    a = np.zeros((h, n_split, d))
    for i in range(h):
        kv = i // g
        x = float(scale) * (k[kv, :seq_len] @ q[i])
        for s in range(n_split):
            lo, hi = s * chunk, min(seq_len, (s + 1) * chunk)
            m[i, s], l[i, s], a[i, s] = state_ref(x[lo:hi], v[kv, lo:hi])
    return m, l, a


def merge_partials_ref(m, l, a, n_valid=None, order=None):
    """N-way merge of split partials into (O, LSE) for one (token, head).

    m, l: [S]; a: [S, d]. Only the first ``n_valid`` partials take part (the
    reducer must use exactly the splits the producer wrote: "Decode attention:
    FlashDecoding, split-K, paged kernels", section "CUDA graphs need the
    split count pinned"). With ``order`` None this is the one-shot reduction
    of that page's stage 2: global maximum over the valid splits, each l_i
    and a_i rescaled by exp(m_i - max), summed, divided once, zero output
    when the total mass is zero. With an explicit ``order`` (a permutation,
    or a nested tuple for a tree) the partials are folded pairwise with
    :func:`merge_ref` in that order instead; the result must not depend on
    it beyond rounding.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    n = m.size if n_valid is None else int(n_valid)
    d = a.shape[-1]
    if order is not None:
        def fold(node):
            if isinstance(node, (tuple, list)):
                st = (EMPTY_M, 0.0, np.zeros(d))
                for child in node:
                    st = merge_ref(st, fold(child))
                return st
            i = int(node)
            return (m[i], l[i], a[i])
        return finalize_ref(fold(order))
    if n == 0:
        return np.zeros(d), -np.inf
    mv, lv, av = m[:n], l[:n], a[:n]
    big = mv.max()
    if np.isneginf(big):
        return np.zeros(d), -np.inf
    w = np.where(np.isneginf(mv), 0.0, np.exp(np.where(np.isneginf(mv), 0.0, mv - big)))
    total = float((w * lv).sum())
    if total == 0.0:
        return np.zeros(d), -np.inf
    o = (w[:, None] * av).sum(axis=0) / total
    return o, big + math.log(total)


def merge_lse_ref(o_a, lse_a, o_b, lse_b):
    """Two-operand merge in (O, LSE) form, elementwise over leading dims.

    o_*: [..., d] normalised outputs over disjoint key ranges, lse_*: [...].
    An LSE of +inf is read as an empty range (-inf), the convention of some
    producers ("Naive attention and the online softmax", section "The base
    case is a NaN factory"). M = max(lse_a, lse_b); the weights
    exp(lse - M) are divided by their sum first, then applied, so the output
    is a convex combination ("Naive attention and the online softmax",
    sections "The state that gets passed around is the log-sum-exp" and
    "Scale first, then multiply"). If both sides are empty the output is
    zeros and LSE -inf. The merged LSE is M + ln(sum of weights).
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    la = np.where(np.isposinf(lse_a), -np.inf, np.asarray(lse_a, dtype=np.float64))
    lb = np.where(np.isposinf(lse_b), -np.inf, np.asarray(lse_b, dtype=np.float64))
    big = np.maximum(la, lb)
    empty = np.isneginf(big)
    safe_big = np.where(empty, 0.0, big)
    ea = np.where(np.isneginf(la), 0.0, np.exp(np.where(np.isneginf(la), 0.0, la - safe_big)))
    eb = np.where(np.isneginf(lb), 0.0, np.exp(np.where(np.isneginf(lb), 0.0, lb - safe_big)))
    tot = ea + eb
    safe_tot = np.where(empty, 1.0, tot)
    pa, pb = ea / safe_tot, eb / safe_tot
    o = o_a * pa[..., None] + o_b * pb[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, big + np.log(safe_tot))
    return o, lse
