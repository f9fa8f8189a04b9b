"""The fp64 ring emulation agrees with the plain definition, whatever the ring
size, chunk sizes or arrival order, and the combine obeys its algebra."""
import itertools

import numpy as np
import pytest

from oracle import attention, combine, ring_share, ring_schedule, block_partial


def _sequence(rng, B, H, T, d):
    return (rng.standard_normal((B, H, T, d)) for _ in range(3))


def _blocks(k, v, N):
    L = k.shape[2] // N
    return {b: (k[:, :, b * L:(b + 1) * L], v[:, :, b * L:(b + 1) * L]) for b in range(N)}


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_ring_size_invariance(causal, N):
    rng = np.random.default_rng(10 + N)
    B, H, T, d = 1, 2, 128, 8
    q, k, v = _sequence(rng, B, H, T, d)
    L = T // N
    blocks = _blocks(k, v, N)
    o_full, lse_full = attention(q, k, v, np.arange(T), np.arange(T), causal)
    for r in range(N):
        qr = q[:, :, r * L:(r + 1) * L]
        o, lse = ring_share(qr, blocks, r, N, L, causal)
        np.testing.assert_allclose(o, o_full[:, :, r * L:(r + 1) * L], atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, lse_full[:, :, r * L:(r + 1) * L], atol=1e-12, rtol=0)


@pytest.mark.parametrize("qc,kc", [(1, 1), (4, 16), (16, 4), (32, 32), (5, 7)])
def test_chunk_invariance(qc, kc):
    rng = np.random.default_rng(20)
    N, L, d = 4, 32, 8
    q, k, v = _sequence(rng, 1, 2, N * L, d)
    blocks = _blocks(k, v, N)
    r = 2
    qr = q[:, :, r * L:(r + 1) * L]
    o_ref, lse_ref = attention(qr, k, v, np.arange(L) + r * L, np.arange(N * L), True)
    o, lse = ring_share(qr, blocks, r, N, L, True, q_chunk=qc, k_chunk=kc)
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_arrival_order_invariance_and_intermediate_state():
    rng = np.random.default_rng(21)
    N, L, d = 6, 16, 8
    q, k, v = _sequence(rng, 1, 1, N * L, d)
    blocks = _blocks(k, v, N)
    r = 4
    qr = q[:, :, r * L:(r + 1) * L]
    q_pos = np.arange(L) + r * L
    o_ref, lse_ref = attention(qr, k, v, q_pos, np.arange(N * L), True)
    for order in [list(rng.permutation(N)) for _ in range(4)]:
        o, lse = ring_share(qr, blocks, r, N, L, True, order=order, q_chunk=8, k_chunk=4)
        np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)
    # after s steps the running state equals the definition on the blocks seen
    sched = ring_schedule(r, N)
    for s in range(1, N + 1):
        seen = [b for b in sched[:s] if b <= r]
        kk = np.concatenate([k[:, :, b * L:(b + 1) * L] for b in seen], axis=2)
        vv = np.concatenate([v[:, :, b * L:(b + 1) * L] for b in seen], axis=2)
        kp = np.concatenate([np.arange(L) + b * L for b in seen])
        o_s, lse_s = attention(qr, kk, vv, q_pos, kp, True)
        o, lse = ring_share(qr, blocks, r, N, L, True, stop_after=s)
        np.testing.assert_allclose(o, o_s, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, lse_s, atol=1e-12, rtol=0)


def test_schedule_reading():
    # step 0 holds the member's own block; blocks arrive from the predecessor
    assert ring_schedule(7, 8) == [7, 6, 5, 4, 3, 2, 1, 0]
    assert ring_schedule(0, 4) == [0, 3, 2, 1]
    for N in (1, 3, 8):
        for r in range(N):
            assert sorted(ring_schedule(r, N)) == list(range(N))


def _partials(rng, n, shape=(2, 3, 9, 4)):
    out = []
    for _ in range(n):
        o = rng.standard_normal(shape)
        lse = rng.standard_normal(shape[:-1]) * 5
        lse[..., 0] = -np.inf          # an empty partial for some rows
        o[..., 0, :] = 0.0
        out.append((o, lse))
    return out


def test_combine_algebra():
    rng = np.random.default_rng(30)
    (a, b, c) = _partials(rng, 3)
    b[1][..., 1] = -np.inf
    b[0][..., 1, :] = 0.0
    ab_c = combine(*combine(*a, *b), *c)
    a_bc = combine(*a, *combine(*b, *c))
    np.testing.assert_allclose(ab_c[0], a_bc[0], atol=1e-14, rtol=0)
    np.testing.assert_allclose(ab_c[1], a_bc[1], atol=1e-14, rtol=0)
    ab, ba = combine(*a, *b), combine(*b, *a)
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-15, rtol=0)
    np.testing.assert_array_equal(ab[1], ba[1])
    ident = (np.zeros_like(a[0]), np.full_like(a[1], -np.inf))
    for x in (combine(*a, *ident), combine(*ident, *a)):
        np.testing.assert_array_equal(x[0], a[0])
        np.testing.assert_array_equal(x[1], a[1])
    # all-empty rows stay the identity, with no NaN
    e = combine(*ident, *ident)
    assert np.isneginf(e[1]).all() and (e[0] == 0).all()


def test_combine_two_halves_is_the_whole():
    rng = np.random.default_rng(31)
    L, d = 50, 8
    q, k, v = (rng.standard_normal((1, 2, L, d)) for _ in range(3))
    pos = np.arange(L)
    whole = attention(q, k, v, pos, pos, True)
    first = attention(q, k[:, :, :20], v[:, :, :20], pos, pos[:20], True)
    second = attention(q, k[:, :, 20:], v[:, :, 20:], pos, pos[20:], True)
    got = combine(*first, *second)
    np.testing.assert_allclose(got[0], whole[0], atol=1e-13, rtol=0)
    np.testing.assert_allclose(got[1], whole[1], atol=1e-13, rtol=0)


def test_block_partial_extreme_scores_no_overflow():
    """Scores near +-700 would overflow a plain exp; the running max keeps the
    blockwise pass finite and equal to the definition."""
    rng = np.random.default_rng(32)
    L, d = 32, 4
    q = rng.standard_normal((1, 1, L, d)) * 40
    k = rng.standard_normal((1, 1, L, d)) * 40
    v = rng.standard_normal((1, 1, L, d))
    pos = np.arange(L)
    o_ref, lse_ref = attention(q, k, v, pos, pos, True)
    o, lse = block_partial(q, k, v, pos, pos, True, q_chunk=8, k_chunk=4)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o, o_ref, atol=1e-10, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=0)
