"""Brute-force attention in pure Python, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see the package docstring). This module exists to
pin :func:`oracle.attention.attention_ref` by an independent computation:
scalar loops, ``math.exp`` and ``math.fsum`` (correctly rounded sums), no
numpy arithmetic. It follows the same definition (the textbook attention of
"Naive attention and the online softmax": logits scaled then masked, softmax
over the visible keys of the row, weighted sum of values; zero output and
LSE -inf for a row with no visible key, "Merge normalized attention without
averaging tile outputs", last paragraph).
"""

import math


def brute_attention(q, k, v, scale, causal=False, key_mask=None, row_mask=None):
    """q: nested lists [B][h][T_q][d]; k, v: [B][h_kv][T_k][d]; masks as
    nested lists of 0/1. Returns (O [B][h][T_q][d], LSE [B][h][T_q]) as
    nested lists of Python floats."""
    n_b, h = len(q), len(q[0])
    t_q, d = len(q[0][0]), len(q[0][0][0])
    h_kv, t_k = len(k[0]), len(k[0][0])
    g = h // h_kv
    out_o, out_lse = [], []
    for b in range(n_b):
        ob, lb = [], []
        for i in range(h):
            kv = i // g
            oi, li = [], []
            for t in range(t_q):
                keys = []
                for j in range(t_k):
                    if causal and j > t + t_k - t_q:
                        continue
                    if key_mask is not None and not key_mask[b][j]:
                        continue
                    if row_mask is not None and not row_mask[b][t]:
                        continue
                    keys.append(j)
                if not keys:
                    oi.append([0.0] * d)
                    li.append(-math.inf)
                    continue
                xs = [scale * math.fsum(q[b][i][t][c] * k[b][kv][j][c] for c in range(d))
                      for j in keys]
                mx = max(xs)
                es = [math.exp(x - mx) for x in xs]
                tot = math.fsum(es)
                oi.append([math.fsum(e * v[b][kv][j][c] for e, j in zip(es, keys)) / tot
                           for c in range(d)])
                li.append(mx + math.log(tot))
            ob.append(oi)
            lb.append(li)
        out_o.append(ob)
        out_lse.append(lb)
    return out_o, out_lse
