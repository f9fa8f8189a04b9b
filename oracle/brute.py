"""Scalar brute-force attention for tiny shapes (pure Python, math.fsum).

Test infrastructure only.  Written independently of ``oracle.attention`` so
that a dropped term, a transposed operand or an off-by-one in the causal mask
there shows up as a disagreement: every score is a fsum of scalar products,
every softmax weight is exp(score - max) / fsum, every output a fsum.
"""
from __future__ import annotations

import math


def brute_attention(q, k, v, q_pos, k_pos, causal, scale=None):
    """q: nested lists [Lq][d]; k, v: [Lk][d]; positions are lists of ints.

    Returns (o [Lq][dv], lse [Lq]) as Python floats; a row that sees no key
    returns zeros and -inf."""
    d = len(q[0])
    sc = (1.0 / math.sqrt(d)) if scale is None else scale
    out, lses = [], []
    for i, qi in enumerate(q):
        scores = []
        for j, kj in enumerate(k):
            if causal and k_pos[j] > q_pos[i]:
                continue
            scores.append((j, sc * math.fsum(a * b for a, b in zip(qi, kj))))
        if not scores:
            out.append([0.0] * len(v[0]))
            lses.append(-math.inf)
            continue
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        z = math.fsum(x for _, x in w)
        out.append([math.fsum(x * v[j][c] for j, x in w) / z for c in range(len(v[0]))])
        lses.append(mx + math.log(z))
    return out, lses
