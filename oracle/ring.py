"""fp64 emulation of the ring schedule, blockwise pass and associative combine.

Test infrastructure only.  This is a second, independent route to the same
numbers as ``oracle.attention``; tests use it to show that ring size, chunk
sizes and arrival order do not change the result, and to pin the combine
algebra.  It follows the method's steps in the order the pages give them:

1. Ring schedule (Ring Attention keyword page, definition): the member keeps
   its query block while key/value blocks circulate.  Reading used here: the
   member receives from its predecessor, so at step s it holds block
   (rank - s) mod N; step 0 is its own block.
2. Blockwise pass (Blockwise RingAttention keyword page, definition; Ring
   Attention with Blockwise Transformers, abstract): the held queries attend
   to the arriving block chunk by chunk, keeping a running max and running
   denominator, never forming the full score matrix of the block.
3. Associative combine (darcstar research page, commentary: online softmax is
   associative, so partials from separate shards combine exactly), with the
   causal mask applied on global positions so seams are exact (same
   commentary, on seams).
"""
from __future__ import annotations

import numpy as np

from .exact import _as64, _scale


def combine(o_a, lse_a, o_b, lse_b):
    """Merge two normalised partials (o, lse) over disjoint key sets.

    Identity element: (0, -inf).  With mu = max(lse_a, lse_b) and
    w_x = exp(lse_x - mu): lse = mu + ln(w_a + w_b),
    o = (w_a o_a + w_b o_b) / (w_a + w_b).  Never forms (-inf) - (-inf)."""
    o_a, lse_a, o_b, lse_b = map(np.asarray, (o_a, lse_a, o_b, lse_b))
    a_live = np.isfinite(lse_a)
    b_live = np.isfinite(lse_b)
    both = a_live & b_live
    mu = np.where(both, np.maximum(lse_a, lse_b), 0.0)
    wa = np.where(both, np.exp(np.where(both, lse_a, 0.0) - mu), 0.0)
    wb = np.where(both, np.exp(np.where(both, lse_b, 0.0) - mu), 0.0)
    z = np.where(both, wa + wb, 1.0)
    lse = np.where(both, mu + np.log(z), np.where(a_live, lse_a, lse_b))
    o_both = (wa[..., None] * o_a + wb[..., None] * o_b) / z[..., None]
    o = np.where(both[..., None], o_both,
                 np.where(a_live[..., None], o_a, np.where(b_live[..., None], o_b, 0.0)))
    return o, lse


def block_partial(q, k, v, q_pos, k_pos, causal, scale=None, q_chunk=None,
                  k_chunk=None):
    """One blockwise pass: queries ``q`` against one key/value block.

    Query chunks are independent; within a query chunk the key chunks are
    visited in order with a running max m, running denominator l and running
    unnormalised output acc.  Returns the normalised partial (o, lse); a row
    that sees no key of this block returns the identity (0, -inf)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    qc = Lq if q_chunk is None else q_chunk
    kc = Lk if k_chunk is None else k_chunk
    sc = _scale(d, scale)
    o = np.zeros((B, H, Lq, v.shape[-1]))
    lse = np.full((B, H, Lq), -np.inf)
    for b in range(B):
        for h in range(H):
            for i0 in range(0, Lq, qc):
                i1 = min(Lq, i0 + qc)
                qt = q[b, h, i0:i1]
                m = np.full(i1 - i0, -np.inf)
                l = np.zeros(i1 - i0)
                acc = np.zeros((i1 - i0, v.shape[-1]))
                for j0 in range(0, Lk, kc):
                    j1 = min(Lk, j0 + kc)
                    s = sc * (qt @ k[b, h, j0:j1].T)
                    if causal:
                        s[k_pos[None, j0:j1] > q_pos[i0:i1, None]] = -np.inf
                    m_new = np.maximum(m, s.max(axis=1))
                    live = np.isfinite(m_new)
                    m_ref = np.where(live, m_new, 0.0)
                    alpha = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - m_ref), 0.0)
                    p = np.exp(s - m_ref[:, None])
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, h, j0:j1]
                    m = m_new
                live = l > 0
                o[b, h, i0:i1] = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
                lse[b, h, i0:i1] = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse


def ring_schedule(rank: int, ring_size: int):
    """Block held at each step: step s holds block (rank - s) mod ring_size."""
    return [(rank - s) % ring_size for s in range(ring_size)]


def ring_share(q, blocks, rank, ring_size, block_len, causal, scale=None,
               q_chunk=None, k_chunk=None, order=None, stop_after=None):
    """One member's share by ring emulation.

    ``blocks`` maps a global block id to its (k, v) arrays; a block that the
    causal mask hides entirely from this member may be missing.  ``order``
    overrides the arrival order (a permutation of block ids);
    ``stop_after`` returns the running state after that many steps.
    Returns (o, lse) of the running accumulator, float64."""
    q = _as64(q)
    B, H, Lq, d = q.shape
    q_pos = np.arange(Lq, dtype=np.int64) + rank * block_len
    o = np.zeros((B, H, Lq, d))
    lse = np.full((B, H, Lq), -np.inf)
    sched = ring_schedule(rank, ring_size) if order is None else list(order)
    for step, kb in enumerate(sched):
        if stop_after is not None and step >= stop_after:
            break
        if causal and kb > rank:
            continue                     # future block: every pair is masked
        k, v = blocks[kb]
        k_pos = np.arange(k.shape[2], dtype=np.int64) + kb * block_len
        o_b, lse_b = block_partial(q, k, v, q_pos, k_pos, causal, scale, q_chunk, k_chunk)
        o, lse = combine(o, lse, o_b, lse_b)
    return o, lse
