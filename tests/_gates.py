"""Parity gates used by the GPU tests, and helpers that evaluate the oracle on
sampled rows of large shares.

Tolerances: fp32 inputs, max |o - ref| <= 1e-4; bf16 inputs with fp32
accumulation, |x - ref| <= 2e-2 + 1e-2 |ref| elementwise for o, dQ, dK, dV;
LSE max-abs <= 1e-3 for both.  Because some outputs are smaller than the
absolute tolerance (an all-zero o would pass it on long shares), every
comparison also bounds the relative Frobenius error (1e-2 for bf16, 1e-5 for
fp32) and rejects NaN / Inf.

Gradients that are sums of many terms of either sign (the feedforward's dx
and weight gradients, up to 16384 terms per entry) are gated against an
error scale instead of |ref|: |x - ref| <= 1e-2 scale (+ a floor of 1e-6 of
the largest scale), where scale is the root-sum-square, over the entry's
terms, of each term's first-order sensitivity to the bf16 roundings of the
intermediates it is formed from (oracle.feedforward_grad_rss).  Each
rounding is a zero-mean relative error the sum does not cancel, so an
entry's error has RMS about 1e-3 times the scale (measured on the CPU with
the kernels' roundings emulated: largest error 6.2e-3 of the scale from one
to 2048 rows), and 1e-2 of it is a median tolerance of 2.2 % of rms(ref).
|ref| itself can be far smaller than the terms, and the sum of their
magnitudes far larger (a tolerance of 22-33 % of rms(ref) at the median),
so neither scales the gate.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def check(name, got, ref, dtype):
    got, ref = _np(got), _np(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref)
    relf = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    if dtype == "fp32":
        assert err.max() <= 1e-4, f"{name}: max abs err {err.max():.3e} > 1e-4"
        assert relf <= 1e-5, f"{name}: rel Frobenius err {relf:.3e} > 1e-5"
    else:
        bad = err > 2e-2 + 1e-2 * np.abs(ref)
        assert not bad.any(), (f"{name}: {bad.sum()} elements outside 2e-2 + 1e-2|ref| "
                               f"(max abs err {err.max():.3e})")
        assert relf <= 1e-2, f"{name}: rel Frobenius err {relf:.3e} > 1e-2"
    return float(err.max()), float(relf)


def check_lse(name, got, ref):
    got, ref = _np(got), _np(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{name}: -inf pattern differs"
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all(), f"{name}: non-finite LSE"
    err = np.abs(got[fin] - ref[fin]).max() if fin.any() else 0.0
    assert err <= 1e-3, f"{name}: LSE max abs err {err:.3e} > 1e-3"
    return float(err)


def seam_rows(L, q_chunk, rng, n_random):
    """Rows at block and chunk seams plus random ones."""
    rows = {0, 1, L - 1, L - 2}
    for c in (32, 64, 128, 256, q_chunk):
        for k in range(c, L, max(c, L // 4)):
            rows.update({k - 1, k})
    rows.update(rng.choice(L, size=min(n_random, L), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < L))


def tile_rows(L, tile, rng, seams=()):
    """One random row inside every `tile`-row tile of a block of L rows (the
    last tile may be ragged), plus the given seam rows."""
    rows = {int(t + rng.integers(min(tile, L - t))) for t in range(0, L, tile)}
    rows.update(r for r in seams if 0 <= r < L)
    return np.array(sorted(rows))


def oracle_rows_per_head(host, rows_of):
    """Oracle o, lse of a member's share on a different row set per head:
    rows_of maps query head -> row indices.  Returns {head: (o [B, n, d],
    lse [B, n])}, one head's keys upcast to float64 at a time."""
    cfg = host.cfg
    L = cfg.block_len
    blocks = sorted(host.kv)
    k_pos = np.concatenate([oracle.positions(b, L) for b in blocks])
    H, Hkv = cfg.heads, host.kv[blocks[0]].shape[2]
    out = {}
    for h, rows in rows_of.items():
        kh = oracle.exact._kv_head(h, H, Hkv)
        k = torch.cat([host.kv[kb][0][:, kh:kh + 1] for kb in blocks], dim=2)
        v = torch.cat([host.kv[kb][1][:, kh:kh + 1] for kb in blocks], dim=2)
        q_pos = oracle.positions(host.rank, L)[rows]
        o, lse = oracle.attention(host.q[:, h:h + 1, rows], k, v, q_pos, k_pos, cfg.causal)
        out[h] = (o[:, 0], lse[:, 0])
    return out


def oracle_rows(host, heads, rows):
    """Oracle o, lse for the given heads and rows of a member's share.

    Works one (b, h) at a time so that only one head's keys are ever upcast
    to float64."""
    cfg = host.cfg
    L = cfg.block_len
    blocks = sorted(host.kv)
    q_pos = oracle.positions(host.rank, L)[rows]
    k_pos = np.concatenate([oracle.positions(b, L) for b in blocks])
    o = np.zeros((cfg.batch, len(heads), len(rows), cfg.head_dim))
    lse = np.zeros((cfg.batch, len(heads), len(rows)))
    H, Hkv = cfg.heads, host.kv[blocks[0]].shape[2]
    for b in range(cfg.batch):
        for i, h in enumerate(heads):
            kh = oracle.exact._kv_head(h, H, Hkv)  # the oracle's own head grouping
            k = torch.cat([host.kv[kb][0, b:b + 1, kh:kh + 1] for kb in blocks], dim=2)
            v = torch.cat([host.kv[kb][1, b:b + 1, kh:kh + 1] for kb in blocks], dim=2)
            qh = host.q[b:b + 1, h:h + 1, rows]
            ob, lb = oracle.attention(qh, k, v, q_pos, k_pos, cfg.causal)
            o[b, i] = ob[0, 0]
            lse[b, i] = lb[0, 0]
    return o, lse


def check_rss(name, got, ref, rss):
    """Elementwise |got - ref| <= 1e-2 * rss + 1e-6 * max(rss) (rss: the
    error scale of each entry, oracle.feedforward_grad_rss), plus the bf16
    relative Frobenius bound and no NaN / Inf."""
    got, ref, rss = _np(got), _np(ref), _np(rss)
    assert got.shape == ref.shape == rss.shape, (name, got.shape, ref.shape, rss.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref)
    tol = 1e-2 * rss + 1e-6 * float(rss.max(initial=0.0))
    bad = err > tol
    assert not bad.any(), (f"{name}: {bad.sum()} elements outside 1e-2 error scale "
                           f"(max err / rss {float((err / np.maximum(rss, 1e-300)).max()):.3e})")
    relf = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert relf <= 1e-2, f"{name}: rel Frobenius err {relf:.3e} > 1e-2"
    return float(err.max()), float(relf)
