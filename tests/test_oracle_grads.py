"""Pins of the oracle's closed-form gradients."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, attention_grads


def _loss(q, k, v, do, qp, kp, causal):
    o, _ = attention(q, k, v, qp, kp, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    rng = np.random.default_rng(40)
    B, H, Lq, Lk, d = 1, 1, 5, 7, 3
    q = rng.standard_normal((B, H, Lq, d))
    k = rng.standard_normal((B, H, Lk, d))
    v = rng.standard_normal((B, H, Lk, d))
    do = rng.standard_normal((B, H, Lq, d))
    qp, kp = np.arange(Lq) + 2, np.arange(Lk)
    dq, dk, dv, _, _ = attention_grads(q, k, v, do, qp, kp, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, qp, kp, causal)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, qp, kp, causal)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_fp64(causal):
    """Independent library route: torch fp64 autograd through the SDPA routine."""
    rng = np.random.default_rng(41)
    B, H, L, d = 1, 2, 48, 16
    arrs = [rng.standard_normal((B, H, L, d)) for _ in range(4)]
    q, k, v, do = arrs
    pos = np.arange(L)
    dq, dk, dv, o, _ = attention_grads(q, k, v, do, pos, pos, causal, row_tile=20)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_gradient_sum_identities():
    """sum_j dV_j = sum_i dO_i (rows of P sum to one) and sum_j dK_j = 0 (each
    row of dS sums to zero over its visible keys), causal mask included."""
    rng = np.random.default_rng(42)
    L, d = 64, 8
    q, k, v, do = (rng.standard_normal((1, 2, L, d)) for _ in range(4))
    pos = np.arange(L)
    dq, dk, dv, _, _ = attention_grads(q, k, v, do, pos, pos, True)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # shifting every key by a constant does not change dQ
    c = rng.standard_normal(d)
    dq2, _, _, _, _ = attention_grads(q, k + c, v, do, pos, pos, True)
    np.testing.assert_allclose(dq2, dq, atol=1e-11)


def test_member_contributions_sum_to_full_gradient():
    """dK/dV of the whole causal sequence equal the sum over ring members of
    each member's contribution from its own query rows."""
    rng = np.random.default_rng(43)
    N, L, d = 4, 16, 8
    T = N * L
    q, k, v, do = (rng.standard_normal((1, 1, T, d)) for _ in range(4))
    pos = np.arange(T)
    dq_f, dk_f, dv_f, _, _ = attention_grads(q, k, v, do, pos, pos, True)
    dk_sum = np.zeros_like(dk_f)
    dv_sum = np.zeros_like(dv_f)
    for r in range(N):
        rows = slice(r * L, (r + 1) * L)
        dq_r, dk_r, dv_r, _, _ = attention_grads(q[:, :, rows], k, v, do[:, :, rows],
                                                  pos[rows], pos, True)
        np.testing.assert_allclose(dq_r, dq_f[:, :, rows], atol=1e-12)
        if r + 1 < N:                                     # future keys untouched
            assert np.abs(dk_r[:, :, (r + 1) * L:]).max() == 0.0
            assert np.abs(dv_r[:, :, (r + 1) * L:]).max() == 0.0
        dk_sum += dk_r
        dv_sum += dv_r
    np.testing.assert_allclose(dk_sum, dk_f, atol=1e-12)
    np.testing.assert_allclose(dv_sum, dv_f, atol=1e-12)


@pytest.mark.parametrize("kv_heads", [1, 2])
def test_shared_kv_heads_autograd_fp64(kv_heads):
    """Shared key/value heads: dK / dV of a key/value head sum over its query
    heads.  Checked against torch fp64 autograd through SDPA's grouped route."""
    rng = np.random.default_rng(43)
    B, H, L, d = 1, 4, 40, 16
    q, do = rng.standard_normal((B, H, L, d)), rng.standard_normal((B, H, L, d))
    k, v = rng.standard_normal((B, kv_heads, L, d)), rng.standard_normal((B, kv_heads, L, d))
    pos = np.arange(L)
    dq, dk, dv, o, _ = attention_grads(q, k, v, do, pos, pos, True, row_tile=16)
    assert dk.shape == k.shape and dv.shape == v.shape
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                          enable_gqa=True)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal,kv_heads", [(True, 2), (False, 1), (True, 4)])
def test_grads_at_chosen_keys_against_torch_autograd(causal, kv_heads):
    """dK / dV of chosen keys (the routine used where the whole dS does not
    fit) against torch fp64 autograd through SDPA with an explicit mask over
    global positions: the rows of member 2 of a ring of blocks of 23 against
    every key up to its own block (past blocks and the diagonal), several row
    tiles with a ragged tail, keys at block seams and inside blocks."""
    from oracle import attention_grads_at_keys
    rng = np.random.default_rng(47 + kv_heads)
    B, H, L, d, rank = 1, 4, 23, 16, 2
    q, do = rng.standard_normal((B, H, L, d)), rng.standard_normal((B, H, L, d))
    Lk = (rank + 1) * L
    k, v = rng.standard_normal((B, kv_heads, Lk, d)), rng.standard_normal((B, kv_heads, Lk, d))
    q_pos, k_pos = rank * L + np.arange(L), np.arange(Lk)
    keys = [0, 5, L - 1, L, 2 * L - 1, 2 * L, 2 * L + 11, Lk - 1]
    dk, dv = attention_grads_at_keys(q, k, v, do, q_pos, k_pos, causal, keys, row_tile=7)
    assert dk.shape == (B, kv_heads, len(keys), d) and dv.shape == dk.shape
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = torch.from_numpy(k_pos[None, :] <= q_pos[:, None]) if causal else None
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                          enable_gqa=True)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dk, tk.grad.numpy()[:, :, keys], atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy()[:, :, keys], atol=1e-12)


def test_grads_at_chosen_keys_ignore_rows_with_no_visible_key():
    """Causal rows placed before every key see nothing and must contribute
    nothing (no NaN from their empty softmax)."""
    from oracle import attention_grads_at_keys
    rng = np.random.default_rng(53)
    q, do = rng.standard_normal((1, 2, 12, 8)), rng.standard_normal((1, 2, 12, 8))
    k, v = rng.standard_normal((1, 2, 10, 8)), rng.standard_normal((1, 2, 10, 8))
    q_pos = np.array([-4, -1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9])
    k_pos = np.arange(10)
    keys = [0, 3, 9]
    dk, dv = attention_grads_at_keys(q, k, v, do, q_pos, k_pos, True, keys, row_tile=5)
    dk2, dv2 = attention_grads_at_keys(q[:, :, 2:], k, v, do[:, :, 2:], q_pos[2:], k_pos, True,
                                       keys, row_tile=5)
    assert np.isfinite(dk).all() and np.isfinite(dv).all()
    np.testing.assert_allclose(dk, dk2, atol=1e-13)
    np.testing.assert_allclose(dv, dv2, atol=1e-13)
