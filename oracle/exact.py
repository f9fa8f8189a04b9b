"""The plain definition of exact (causal) softmax attention, in float64.

Test infrastructure only (see the package docstring).

Ring Attention keyword page (definition) and the Ring Attention with
Blockwise Transformers abstract state that the ring computes ordinary
self-attention exactly, with no approximation; the darcstar commentary adds
that the causal masking and the softmax normaliser have to stay exact
across chunk seams.  The oracle therefore writes out the definition
directly:

    S_ij   = scale * <q_i, k_j>                 (scale defaults to 1/sqrt(d))
    allowed(i, j) = (not causal) or kpos_j <= qpos_i      (global positions)
    LSE_i  = ln sum_{j allowed} exp(S_ij)
    O_i    = sum_{j allowed} exp(S_ij - LSE_i) v_j

and materialises S one tile of query rows at a time (a plain memory bound,
not a reordering of the arithmetic: each row is computed whole).  A row with
no allowed key gets O_i = 0 and LSE_i = -inf.

Shared key/value heads (MQA / GQA, named on the kongchang "Ring Attention"
knowledge page, facts list, as sharing key-value heads): with H query heads
and Hkv key/value heads, query head h uses key/value head h // (H // Hkv), and
the gradient of a shared key/value head is the sum over the query heads that
use it.  Hkv == H is ordinary multi-head attention.
"""
from __future__ import annotations

import numpy as np


def positions(block: int, block_len: int, length: int | None = None) -> np.ndarray:
    """Global token positions of a contiguous block (member ``block`` owns
    tokens block*block_len ... block*block_len + block_len - 1)."""
    n = block_len if length is None else length
    return np.arange(n, dtype=np.int64) + np.int64(block) * np.int64(block_len)


def _as64(x) -> np.ndarray:
    if hasattr(x, "detach"):          # torch tensor (bf16 has no numpy dtype)
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _scale(d: int, scale: float | None) -> float:
    return 1.0 / np.sqrt(d) if scale is None else float(scale)


def _check_heads(H: int, k) -> int:
    """The key/value head count, which must divide the query head count."""
    Hkv = k.shape[1]
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"{Hkv} key/value heads do not divide {H} query heads")
    return Hkv


def _kv_head(h: int, H: int, Hkv: int) -> int:
    """Key/value head of query head h: consecutive groups of H / Hkv."""
    return h // (H // Hkv)


def _scores(qt, k, qpos_t, kpos, causal, scale):
    s = scale * (qt @ k.T)
    if causal:
        s[kpos[None, :] > qpos_t[:, None]] = -np.inf
    return s


def attention(q, k, v, q_pos, k_pos, causal: bool, scale: float | None = None,
              row_tile: int = 256):
    """Exact attention of the rows ``q`` against the keys ``k`` / values ``v``.

    q: [B, H, Lq, d]; k, v: [B, Hkv, Lk, d] with Hkv dividing H; q_pos: [Lq];
    k_pos: [Lk] global positions.  Returns (o [B, H, Lq, d], lse [B, H, Lq])
    in float64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    B, H, Lq, d = q.shape
    Hkv = _check_heads(H, k)
    sc = _scale(d, scale)
    o = np.zeros((B, H, Lq, v.shape[-1]))
    lse = np.full((B, H, Lq), -np.inf)
    for b in range(B):
        for h in range(H):
            kh = _kv_head(h, H, Hkv)
            for r0 in range(0, Lq, row_tile):
                r1 = min(Lq, r0 + row_tile)
                s = _scores(q[b, h, r0:r1], k[b, kh], q_pos[r0:r1], k_pos, causal, sc)
                m = s.max(axis=1)
                live = np.isfinite(m)
                m_safe = np.where(live, m, 0.0)
                e = np.exp(s - m_safe[:, None])
                l = e.sum(axis=1)
                num = e @ v[b, kh]
                o[b, h, r0:r1] = np.where(live[:, None], num / np.where(live, l, 1.0)[:, None], 0.0)
                lse[b, h, r0:r1] = np.where(live, m_safe + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse


def attention_grads(q, k, v, do, q_pos, k_pos, causal: bool,
                    scale: float | None = None, row_tile: int = 256):
    """Exact gradients of sum(dO * O) with respect to q, k and v.

    With P = softmax(S + M) row-wise and delta_i = <dO_i, O_i>:
        dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),
        dQ = scale * dS K,  dK = scale * dS^T Q.
    With shared key/value heads, dK and dV of a key/value head sum the
    contributions of its query heads.  Returns (dq, dk, dv, o, lse), all
    float64; dk and dv have the key/value head count."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    B, H, Lq, d = q.shape
    Hkv = _check_heads(H, k)
    sc = _scale(d, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros((B, H, Lq, v.shape[-1]))
    lse = np.full((B, H, Lq), -np.inf)
    for b in range(B):
        for h in range(H):
            kh = _kv_head(h, H, Hkv)
            for r0 in range(0, Lq, row_tile):
                r1 = min(Lq, r0 + row_tile)
                s = _scores(q[b, h, r0:r1], k[b, kh], q_pos[r0:r1], k_pos, causal, sc)
                m = s.max(axis=1)
                live = np.isfinite(m)
                m_safe = np.where(live, m, 0.0)
                e = np.exp(s - m_safe[:, None])
                l = np.where(live, e.sum(axis=1), 1.0)
                p = e / l[:, None]
                p[~live] = 0.0
                ot = p @ v[b, kh]
                o[b, h, r0:r1] = ot
                lse[b, h, r0:r1] = np.where(live, m_safe + np.log(l), -np.inf)
                dot = do[b, h, r0:r1]
                delta = (dot * ot).sum(axis=1)
                dp = dot @ v[b, kh].T
                ds = p * (dp - delta[:, None])
                dq[b, h, r0:r1] = sc * (ds @ k[b, kh])
                dk[b, kh] += sc * (ds.T @ q[b, h, r0:r1])
                dv[b, kh] += p.T @ dot
    return dq, dk, dv, o, lse


def attention_grads_at_keys(q, k, v, do, q_pos, k_pos, causal: bool, keys,
                            scale: float | None = None, row_tile: int = 256):
    """dK and dV of the chosen keys only (``keys``: indices into the key
    axis), for shares whose full dS does not fit in memory.

    The same closed form as ``attention_grads``.  First the log-sum-exp
    LSE_i and delta_i = <dO_i, O_i> of every row (each row computed whole,
    one tile of rows at a time); then, for each chosen key j,
        P_ij = exp(S_ij - LSE_i),
        dV_j = sum_i P_ij dO_i,
        dK_j = scale * sum_i P_ij (<dO_i, v_j> - delta_i) q_i,
    summed over the query heads that share key/value head of j.  Rows with
    no allowed key contribute nothing.  Returns (dk, dv), float64
    [B, Hkv, len(keys), d]."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    B, H, Lq, d = q.shape
    Hkv = _check_heads(H, k)
    sc = _scale(d, scale)
    dk = np.zeros((B, Hkv, len(keys), k.shape[-1]))
    dv = np.zeros((B, Hkv, len(keys), v.shape[-1]))
    for b in range(B):
        for h in range(H):
            kh = _kv_head(h, H, Hkv)
            lse = np.full(Lq, -np.inf)
            delta = np.zeros(Lq)
            for r0 in range(0, Lq, row_tile):       # every row's LSE and delta
                r1 = min(Lq, r0 + row_tile)
                s = _scores(q[b, h, r0:r1], k[b, kh], q_pos[r0:r1], k_pos, causal, sc)
                m = s.max(axis=1)
                live = np.isfinite(m)
                m_safe = np.where(live, m, 0.0)
                e = np.exp(s - m_safe[:, None])
                l = np.where(live, e.sum(axis=1), 1.0)
                ot = (e @ v[b, kh]) / l[:, None]
                ot[~live] = 0.0
                lse[r0:r1] = np.where(live, m_safe + np.log(l), -np.inf)
                delta[r0:r1] = (do[b, h, r0:r1] * ot).sum(axis=1)
            ks, vs, kp = k[b, kh][keys], v[b, kh][keys], k_pos[keys]
            for r0 in range(0, Lq, row_tile):       # the chosen keys' columns
                r1 = min(Lq, r0 + row_tile)
                live = np.isfinite(lse[r0:r1])
                s = _scores(q[b, h, r0:r1], ks, q_pos[r0:r1], kp, causal, sc)
                p = np.exp(s - np.where(live, lse[r0:r1], 0.0)[:, None])
                p[~live] = 0.0
                dot = do[b, h, r0:r1]
                ds = p * (dot @ vs.T - delta[r0:r1, None])
                dk[b, kh] += sc * (ds.T @ q[b, h, r0:r1])
                dv[b, kh] += p.T @ dot
    return dk, dv
