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


def _empty(d):
    """The state of no keys: reference -inf, mass 0, numerator 0."""
    return EMPTY_M, 0.0, np.zeros(d)


def state_ref(scores, values):
    """Partial state (m, l, a) of one block of keys.

    scores: [n] logits of the block (-inf marks an excluded key); values:
    [n, d]. The reference m is the largest visible logit, and every weight
    exp(x - m) lies in (0, 1] ("The Online Softmax Recurrence", section "The
    recurrence"). With no visible key the reference would be -inf and
    x - m would read -inf - (-inf), so that case is decided before any
    subtraction and gives the empty state ("The Online Softmax Recurrence",
    section "Where it breaks"; "Merge normalized attention without averaging
    tile outputs", paragraph on fully masked tiles).
    """
    logits = np.asarray(scores, dtype=np.float64)
    rows = np.asarray(values, dtype=np.float64)
    visible = ~np.isneginf(logits)
    if not visible.any():
        return _empty(rows.shape[-1])
    ref = float(logits[visible].max())
    weights = np.exp(logits - ref)          # excluded keys: exp(-inf) = 0
    return ref, float(weights.sum()), weights @ rows


def _combine(states):
    """Fold any number of states of disjoint key sets into one.

    The combined reference is the largest of the inputs' references; input
    i enters with the factor exp(m_i - m), which is in [0, 1], applied to
    its mass and its numerator ("Merge normalized attention without
    averaging tile outputs", paragraph on disjoint nonempty tiles; "The
    Online Softmax Recurrence", section "The recurrence"). Inputs whose
    reference is -inf (empty) get the factor 0 without forming
    -inf - (-inf); if every input is empty the result is the empty state
    ("Merge normalized attention without averaging tile outputs", paragraph
    on fully masked tiles).
    """
    refs = np.array([float(s[0]) for s in states])
    width = np.asarray(states[0][2], dtype=np.float64).shape[-1]
    live = ~np.isneginf(refs)
    if not live.any():
        return _empty(width)
    top = float(refs[live].max())
    factor = [math.exp(r - top) if ok else 0.0 for r, ok in zip(refs, live)]
    mass = 0.0
    numer = np.zeros(width)
    for f, (_, l_i, a_i) in zip(factor, states):
        mass = mass + l_i * f
        numer = numer + np.asarray(a_i, dtype=np.float64) * f
    return top, mass, numer


def merge_ref(a, b):
    """Merge two states of disjoint key sets (the two-input case of the
    fold above); the result does not depend on the order of a and b."""
    return _combine([a, b])


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
    section (3) "The online recurrence", carried to the output in section
    "Extending the recurrence to the output": the running reference after a
    block is the largest logit seen so far; when it rises from r to r', the
    mass and the output accumulator collected so far are multiplied by
    exp(r - r') before the block's weights exp(x - r') are added. Before
    any visible key the state is empty (reference -inf): a block that leaves
    it there adds nothing, and the first block that does not gets the decay
    0 in place of exp(-inf - r').

    Returns the final state (m, l, O~); divide once at the end with
    :func:`finalize_ref`.
    """
    logits = np.asarray(scores, dtype=np.float64)
    rows = np.asarray(values, dtype=np.float64)
    starts = range(0, logits.size, block)
    # running reference after each block: a prefix maximum of block maxima
    refs = np.maximum.accumulate([float(logits[s:s + block].max()) for s in starts]) if logits.size else []
    ref, mass, acc = EMPTY_M, 0.0, np.zeros(rows.shape[-1])
    for s, r_new in zip(starts, refs):
        r_new = float(r_new)
        if np.isneginf(r_new):
            continue
        decay = 0.0 if np.isneginf(ref) else math.exp(ref - r_new)
        w = np.exp(logits[s:s + block] - r_new)
        mass = decay * mass + float(w.sum())
        acc = decay * acc + w @ rows[s:s + block]
        ref = r_new
    return ref, mass, acc


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
