"""Plant plausible slips in the oracle (on the CPU) and check that the pins
catch every one of them.  The slips are monkeypatched into the oracle module
for the duration of one test only."""
import numpy as np
import pytest

import oracle.exact as oa
from oracle.brute import brute_attention


def _pin_brute(attn):
    """The brute-force pin of test_oracle_pins, as a boolean."""
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((1, 1, n, 4)) for n in (6, 9, 9))
    qp, kp = np.arange(6) + 3, np.arange(9)
    ok = True
    for causal in (False, True):
        o, lse = attn(q, k, v, qp, kp, causal, scale=0.6)
        ob, lb = brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                 qp.tolist(), kp.tolist(), causal, scale=0.6)
        ok &= np.allclose(o[0, 0], ob, atol=1e-12) and np.allclose(lse[0, 0], lb, atol=1e-12)
    return ok


def _diag_excluded(qt, k, qpos_t, kpos, causal, scale):
    s = scale * (qt @ k.T)
    if causal:
        s[kpos[None, :] >= qpos_t[:, None]] = -np.inf
    return s


_real_scores = oa._scores


def _no_scale(qt, k, qpos_t, kpos, causal, scale):
    return _real_scores(qt, k, qpos_t, kpos, causal, 1.0)


def _local_positions(qt, k, qpos_t, kpos, causal, scale):
    # a classic seam bug: mask on local instead of global positions
    s = scale * (qt @ k.T)
    if causal:
        local_q = np.arange(len(qpos_t))
        s[np.arange(len(kpos))[None, :] > local_q[:, None]] = -np.inf
    return s


def _sign_flip(qt, k, qpos_t, kpos, causal, scale):
    return -_real_scores(qt, k, qpos_t, kpos, causal, scale)


def _reversed_keys(qt, k, qpos_t, kpos, causal, scale):
    # keys paired with the wrong positions (reversed order)
    return _real_scores(qt, k[::-1], qpos_t, kpos, causal, scale)


@pytest.mark.parametrize("slip", [_diag_excluded, _no_scale, _local_positions,
                                  _sign_flip, _reversed_keys])
def test_planted_slip_is_caught(monkeypatch, slip):
    assert _pin_brute(oa.attention), "the unmodified oracle must pass its pin"
    monkeypatch.setattr(oa, "_scores", slip)
    assert not _pin_brute(oa.attention), f"pin missed planted slip {slip.__name__}"


def test_planted_missing_max_shift_term_is_caught(monkeypatch):
    """Forgetting to add the max back into the LSE leaves O intact; the LSE
    comparison must still fail."""
    def bad_attention(q, k, v, q_pos, k_pos, causal, scale=None, row_tile=256):
        o, lse = oa.attention(q, k, v, q_pos, k_pos, causal, scale, row_tile)
        # subtract each row's max score back out, as a buggy LSE would
        s = (scale if scale is not None else 1 / np.sqrt(q.shape[-1])) * np.einsum(
            "bhid,bhjd->bhij", q, k)
        if causal:
            s = np.where(np.asarray(k_pos)[None, None, None, :] > np.asarray(q_pos)[None, None, :, None], -np.inf, s)
        return o, lse - s.max(axis=-1)
    assert not _pin_brute(bad_attention)


def test_planted_interleaved_kv_groups_are_caught(monkeypatch):
    """Query head h must read key/value head h // (H / Hkv) (contiguous groups);
    the interleaved h % Hkv slip must fail the library grouped-head pin."""

    from tests.test_oracle_pins import test_shared_kv_heads_library_sdpa_fp64 as pin
    pin(2)  # the unmodified oracle passes
    monkeypatch.setattr(oa, "_kv_head", lambda h, H, Hkv: h % Hkv)
    with pytest.raises(AssertionError):
        pin(2)


@pytest.mark.parametrize("slip", [_diag_excluded, _no_scale, _local_positions, _sign_flip])
def test_planted_slip_fails_the_chosen_keys_pin(monkeypatch, slip):
    """The chosen-keys gradient routine shares the score helper: each slip
    there must also fail its autograd pin."""
    from tests.test_oracle_grads import test_grads_at_chosen_keys_against_torch_autograd as pin
    pin(True, 2)  # the unmodified oracle passes
    monkeypatch.setattr(oa, "_scores", slip)
    with pytest.raises(AssertionError):
        pin(True, 2)


def test_planted_interleaved_kv_groups_fail_the_chosen_keys_pin(monkeypatch):
    from tests.test_oracle_grads import test_grads_at_chosen_keys_against_torch_autograd as pin
    pin(True, 2)
    monkeypatch.setattr(oa, "_kv_head", lambda h, H, Hkv: h % Hkv)
    with pytest.raises(AssertionError):
        pin(True, 2)
