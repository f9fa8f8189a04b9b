"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each pin is chosen so that a plausible slip in ``oracle.attention`` (a dropped
scale, a transposed operand, the causal diagonal excluded, the max shift
applied to only one side) fails at least one of them; ``test_oracle_teeth``
plants such slips and checks that they are caught.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention, positions
from oracle.brute import brute_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(causal, seed):
    rng = np.random.default_rng(seed)
    B, H, Lq, Lk, d = 2, 2, 7, 11, 5
    q, k, v = _rand(rng, B, H, Lq, d), _rand(rng, B, H, Lk, d), _rand(rng, B, H, Lk, 3)
    # arbitrary (non-contiguous) global positions stress the seam rule
    q_pos = np.sort(rng.choice(40, Lq, replace=False))
    k_pos = np.sort(rng.choice(40, Lk, replace=False))
    o, lse = attention(q, k, v, q_pos, k_pos, causal, scale=0.7, row_tile=3)
    for b in range(B):
        for h in range(H):
            ob, lb = brute_attention(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(),
                                     q_pos.tolist(), k_pos.tolist(), causal, scale=0.7)
            np.testing.assert_allclose(o[b, h], np.array(ob), atol=1e-13, rtol=0)
            np.testing.assert_array_equal(np.isinf(lse[b, h]), np.isinf(lb))
            fin = np.isfinite(lb)
            np.testing.assert_allclose(lse[b, h][fin], np.array(lb)[fin], atol=1e-13, rtol=0)


def _frac(s):
    return float(Fraction(s))


def test_closed_form_golden():
    with open(os.path.join(GOLDEN, "closed_form_small.json")) as f:
        g = json.load(f)
    a = np.array(g["a"], dtype=np.float64)
    vals = np.array(g["values"], dtype=np.float64)
    for case in g["cases"]:
        k = np.stack([np.log(a), np.zeros_like(a)], axis=1)[None, None]
        v = vals[None, None]
        nq = len(case["q_pos"])
        q = np.tile(np.array([case["c"], 0.0]), (nq, 1))[None, None]
        o, lse = attention(q, k, v, case["q_pos"], case["k_pos"], case["causal"], scale=g["scale"])
        want_o = np.array([[_frac(x) for x in row] for row in case["o"]])
        np.testing.assert_allclose(o[0, 0], want_o, atol=1e-14, rtol=0, err_msg=case["name"])
        for i, arg in enumerate(case["lse_of"]):
            if case["name"].endswith("sees nothing"):
                assert lse[0, 0, i] == -np.inf
            else:
                assert abs(lse[0, 0, i] - math.log(_frac(arg))) < 1e-14, case["name"]


@pytest.mark.parametrize("causal", [False, True])
def test_library_sdpa_fp64(causal):
    """Special case that reduces to a library routine: torch SDPA, fp64 CPU."""
    rng = np.random.default_rng(5)
    B, H, L, d = 1, 3, 96, 32
    q, k, v = _rand(rng, B, H, L, d), _rand(rng, B, H, 2 * L, d), _rand(rng, B, H, 2 * L, d)
    q_pos = positions(1, L)            # member 1 of a ring with block length L
    k_pos = np.arange(2 * L)           # blocks 0 and 1
    o, lse = attention(q, k, v, q_pos, k_pos, causal, row_tile=40)
    mask = torch.ones(L, 2 * L, dtype=torch.bool)
    if causal:
        mask = torch.from_numpy(k_pos[None, :] <= q_pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    s = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) / math.sqrt(d)
    s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    """Extract P itself by attending to one-hot values: rows sum to 1, P >= 0,
    and masked entries are exactly 0."""
    rng = np.random.default_rng(3)
    L, d = 24, 8
    q, k = _rand(rng, 1, 1, L, d), _rand(rng, 1, 1, L, d)
    v = np.eye(L)[None, None]
    p, _ = attention(q, k, v, np.arange(L), np.arange(L), causal)
    p = p[0, 0]
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14, rtol=0)
    assert (p >= 0).all()
    if causal:
        assert (p[np.triu_indices(L, 1)] == 0).all()
        assert (np.diag(p) > 0).all()        # the diagonal is visible


def test_causal_independence():
    """Perturbing keys/values after position i leaves row i bitwise unchanged."""
    rng = np.random.default_rng(4)
    L, d = 64, 16
    q, k, v = _rand(rng, 1, 2, L, d), _rand(rng, 1, 2, L, d), _rand(rng, 1, 2, L, d)
    pos = np.arange(L)
    o, lse = attention(q, k, v, pos, pos, True)
    cut = 37
    k2, v2 = k.copy(), v.copy()
    k2[:, :, cut + 1:] += 5 * _rand(rng, 1, 2, L - cut - 1, d)
    v2[:, :, cut + 1:] -= 3 * _rand(rng, 1, 2, L - cut - 1, d)
    o2, lse2 = attention(q, k2, v2, pos, pos, True)
    np.testing.assert_array_equal(o[:, :, :cut + 1], o2[:, :, :cut + 1])
    np.testing.assert_array_equal(lse[:, :, :cut + 1], lse2[:, :, :cut + 1])
    assert not np.allclose(o[:, :, cut + 1:], o2[:, :, cut + 1:])


def test_closed_forms():
    rng = np.random.default_rng(6)
    L, d = 40, 16
    pos = np.arange(L) + 3 * L                     # a member far into the ring
    q, k, v = _rand(rng, 1, 1, L, d), _rand(rng, 1, 1, L, d), _rand(rng, 1, 1, L, d)
    # Q = 0: uniform weights over the visible keys
    o, lse = attention(np.zeros_like(q), k, v, pos, pos, True)
    counts = np.arange(1, L + 1)
    np.testing.assert_allclose(o[0, 0], np.cumsum(v[0, 0], axis=0) / counts[:, None], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(counts), atol=1e-14)
    # V = 1: every output is exactly one
    o, _ = attention(q, k, np.ones_like(v), pos, pos, True)
    np.testing.assert_allclose(o, 1.0, atol=1e-14)
    # the first row of the sequence sees only itself
    o, lse = attention(q, k, v, np.arange(L), np.arange(L), True)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 0] - q[0, 0, 0] @ k[0, 0, 0] / math.sqrt(d)) < 1e-13
    # shifting every key by c leaves O and shifts LSE_i by scale * <q_i, c>
    c = _rand(rng, d)
    o1, l1 = attention(q, k, v, pos, pos, True)
    o2, l2 = attention(q, k + c, v, pos, pos, True)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, (q[0, 0] @ c / math.sqrt(d))[None, None], atol=1e-12)
    # linearity in V
    v2 = _rand(rng, 1, 1, L, d)
    oa, _ = attention(q, k, 2 * v - 3 * v2, pos, pos, True)
    ob, _ = attention(q, k, v, pos, pos, True)
    oc, _ = attention(q, k, v2, pos, pos, True)
    np.testing.assert_allclose(oa, 2 * ob - 3 * oc, atol=1e-12)
    # without the mask, permuting the keys (with their values) changes nothing
    perm = rng.permutation(L)
    o1, l1 = attention(q, k, v, pos, pos, False)
    o2, l2 = attention(q, k[:, :, perm], v[:, :, perm], pos, pos, False)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)


@pytest.mark.parametrize("kv_heads", [1, 2])
def test_shared_kv_heads_library_sdpa_fp64(kv_heads):
    """Shared key/value heads (MQA / GQA): the oracle against torch SDPA's own
    grouped-head route (enable_gqa), fp64 CPU, causal over global positions."""
    rng = np.random.default_rng(6)
    B, H, L, d = 2, 4, 64, 16
    q = _rand(rng, B, H, L, d)
    k, v = _rand(rng, B, kv_heads, 2 * L, d), _rand(rng, B, kv_heads, 2 * L, d)
    q_pos, k_pos = positions(1, L), np.arange(2 * L)
    o, lse = attention(q, k, v, q_pos, k_pos, True, row_tile=24)
    mask = torch.from_numpy(k_pos[None, :] <= q_pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask,
        enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    # query head h reads key/value head h // (H // kv_heads): a contiguous group
    kk = torch.from_numpy(k).repeat_interleave(H // kv_heads, dim=1)
    s = torch.from_numpy(q) @ kk.transpose(-1, -2) / math.sqrt(d)
    s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)


def test_decode_rows_after_every_key_library_sdpa_fp64():
    """Decode-shaped rows (a few new queries placed after every key) under the
    causal mask reduce to unmasked attention: torch SDPA without a mask, fp64
    CPU, with grouped key/value heads and three blocks of keys."""
    rng = np.random.default_rng(8)
    B, H, Hkv, Lq, Lk, d = 2, 8, 2, 3, 50, 16
    q = _rand(rng, B, H, Lq, d)
    k, v = _rand(rng, B, Hkv, 3 * Lk, d), _rand(rng, B, Hkv, 3 * Lk, d)
    k_pos = np.arange(3 * Lk)
    q_pos = positions(3, Lk, Lq)          # after blocks 0, 1 and 2
    o, lse = attention(q, k, v, q_pos, k_pos, True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    kk = torch.from_numpy(k).repeat_interleave(H // Hkv, dim=1)
    s = torch.from_numpy(q) @ kk.transpose(-1, -2) / math.sqrt(d)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)
    o_nc, lse_nc = attention(q, k, v, q_pos, k_pos, False)
    np.testing.assert_array_equal(o, o_nc)
    np.testing.assert_array_equal(lse, lse_nc)
