"""Pins of the blockwise-feedforward oracle (oracle/ffn.py) against facts fixed
outside it: printed values of the normal distribution function, a scalar
brute-force evaluation, torch's fp64 linear and GELU (library routines), and
the identities of a position-wise map.  The last test plants slips in the
oracle and checks that the pins catch them."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.ffn as of
from oracle import feedforward, gelu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, rows, d_model, d_ff):
    return (rng.standard_normal((rows, d_model)),
            rng.standard_normal((d_ff, d_model)) / math.sqrt(d_model),
            rng.standard_normal((d_model, d_ff)) / math.sqrt(d_ff))


def _pin_table(ffn=None):
    """With W1 = W2 = identity, FFN(x) = GELU(x) = x Phi(x) elementwise."""
    ffn = ffn or feedforward
    g = json.load(open(os.path.join(GOLDEN, "ffn_gelu_table.json")))
    z = np.array([float(k) for k in g["phi"]] + [-float(k) for k in g["phi"]])
    phi = np.array(list(g["phi"].values()) + [1.0 - p for p in g["phi"].values()])
    n = len(z)
    got = ffn(z[None, :], np.eye(n), np.eye(n))[0]
    return np.abs(got - z * phi).max() <= 1e-14


def _brute(x, w1, w2):
    out = []
    for row in x:
        h = []
        for wf in w1:
            a = math.fsum(xi * wi for xi, wi in zip(row, wf))
            h.append(a * 0.5 * (1.0 + math.erf(a / math.sqrt(2.0))))
        out.append([math.fsum(hf * w for hf, w in zip(h, wc)) for wc in w2])
    return np.array(out)


def _pin_brute(ffn=None):
    ffn = ffn or feedforward
    rng = np.random.default_rng(1)
    x, w1, w2 = _rand(rng, 5, 4, 7)
    return np.abs(ffn(x, w1, w2) - _brute(x.tolist(), w1.tolist(), w2.tolist())).max() <= 1e-13


def _pin_torch(ffn=None, d_model=16, d_ff=40):
    ffn = ffn or feedforward
    rng = np.random.default_rng(2)
    x, w1, w2 = _rand(rng, 33, d_model, d_ff)
    t = [torch.from_numpy(a) for a in (x, w1, w2)]
    ref = torch.nn.functional.linear(
        torch.nn.functional.gelu(torch.nn.functional.linear(t[0], t[1]), approximate="none"), t[2])
    return np.abs(ffn(x, w1, w2) - ref.numpy()).max() <= 1e-12


def test_gelu_matches_the_normal_table():
    assert _pin_table()


def test_gelu_special_values():
    assert gelu(0.0) == 0.0
    assert abs(gelu(40.0) - 40.0) < 1e-12          # Phi -> 1
    assert abs(gelu(-40.0)) < 1e-12                # Phi -> 0


def test_brute_force_tiny():
    assert _pin_brute()


def test_library_torch_fp64():
    assert _pin_torch()


def test_position_wise_and_blockwise():
    """Rows are independent: permuting rows permutes outputs, and chunks of
    rows evaluated separately give the same rows (the blockwise form)."""
    rng = np.random.default_rng(3)
    x, w1, w2 = _rand(rng, 50, 8, 24)
    full = feedforward(x, w1, w2)
    perm = rng.permutation(50)
    np.testing.assert_array_equal(feedforward(x[perm], w1, w2), full[perm])
    chunks = np.concatenate([feedforward(x[i:i + 16], w1, w2) for i in range(0, 50, 16)])
    np.testing.assert_array_equal(chunks, full)


def test_linear_in_w2():
    rng = np.random.default_rng(4)
    x, w1, w2 = _rand(rng, 9, 8, 12)
    w2b = rng.standard_normal(w2.shape)
    lhs = feedforward(x, w1, 2.0 * w2 - 0.5 * w2b)
    rhs = 2.0 * feedforward(x, w1, w2) - 0.5 * feedforward(x, w1, w2b)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12, rtol=0)


def test_shape_mismatch_rejected():
    with pytest.raises(ValueError):
        feedforward(np.zeros((2, 4)), np.zeros((6, 4)), np.zeros((6, 4)))


def _tanh_gelu(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def _relu(z):
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0)


_real_gelu = of.gelu


def _sign_slip(z):
    return _real_gelu(-np.asarray(z, dtype=np.float64))


@pytest.mark.parametrize("slip", [_tanh_gelu, _relu, _sign_slip], ids=["tanh-form", "relu",
                                                                      "sign"])
def test_planted_activation_slip_is_caught(monkeypatch, slip):
    assert _pin_table() and _pin_brute() and _pin_torch()
    monkeypatch.setattr(of, "gelu", slip)
    assert not (_pin_table() and _pin_brute() and _pin_torch())


@pytest.mark.parametrize("which", ["w1", "w2"])
def test_planted_untransposed_weight_is_caught(which):
    """A weight used in the (in, out) instead of the (out, in) layout: with
    square weights the shapes still chain, so only the values can tell."""
    def slipped(x, w1, w2):
        x, w1, w2 = of._as64(x), of._as64(w1), of._as64(w2)
        a = x @ (w1 if which == "w1" else w1.T)
        return of.gelu(a) @ (w2 if which == "w2" else w2.T)
    assert _pin_torch(d_model=16, d_ff=16)
    assert not _pin_torch(slipped, d_model=16, d_ff=16)


# ---- gradients -------------------------------------------------------------

from oracle import feedforward_grads, gelu_grad  # noqa: E402


def _pin_grad_table(gg=None):
    """GELU'(z) = Phi(z) + z phi(z) at the printed table points and at -z."""
    gg = gg or gelu_grad
    g = json.load(open(os.path.join(GOLDEN, "ffn_gelu_table.json")))
    ok = True
    for k, phi in g["phi"].items():
        z, dens = float(k), g["pdf"][k]
        ok &= abs(float(gg(z)) - (phi + z * dens)) <= 1e-14
        ok &= abs(float(gg(-z)) - ((1.0 - phi) - z * dens)) <= 1e-14
    return ok


def _pin_grads_autograd(grads=None, d_model=12, d_ff=20):
    grads = grads or feedforward_grads
    rng = np.random.default_rng(11)
    x, w1, w2 = _rand(rng, 17, d_model, d_ff)
    dout = rng.standard_normal((17, d_model))
    t = [torch.from_numpy(a).requires_grad_(True) for a in (x, w1, w2)]
    out = torch.nn.functional.linear(
        torch.nn.functional.gelu(torch.nn.functional.linear(t[0], t[1]), approximate="none"), t[2])
    (out * torch.from_numpy(dout)).sum().backward()
    got = grads(x, w1, w2, dout)
    return all(np.abs(g - r.grad.numpy()).max() <= 1e-12 for g, r in zip(got, t))


def test_gelu_grad_matches_the_normal_table():
    assert _pin_grad_table()


def test_grads_torch_autograd_fp64():
    assert _pin_grads_autograd()


def test_grads_central_differences():
    rng = np.random.default_rng(12)
    x, w1, w2 = _rand(rng, 4, 3, 5)
    dout = rng.standard_normal((4, 3))
    dx, dw1, dw2 = feedforward_grads(x, w1, w2, dout)
    eps = 1e-6

    def loss(a, b, c):
        return float((dout * feedforward(a, b, c)).sum())
    for arr, grad, which in ((x, dx, 0), (w1, dw1, 1), (w2, dw2, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args = [x.copy(), w1.copy(), w2.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            num[idx] = (up - loss(*args)) / (2 * eps)
        np.testing.assert_allclose(grad, num, atol=1e-7, rtol=0)


def test_hidden_units_are_independent():
    """dW1 rows and dW2 columns of a set of hidden units come from those
    units alone (the full-size GPU test samples them this way)."""
    rng = np.random.default_rng(13)
    x, w1, w2 = _rand(rng, 30, 8, 40)
    dout = rng.standard_normal((30, 8))
    _, dw1, dw2 = feedforward_grads(x, w1, w2, dout)
    fs = np.array([0, 7, 39])
    _, s1, s2 = feedforward_grads(x, w1[fs], w2[:, fs], dout)
    np.testing.assert_allclose(s1, dw1[fs], atol=1e-13, rtol=0)
    np.testing.assert_allclose(s2, dw2[:, fs], atol=1e-13, rtol=0)


def _grad_missing_density(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + of.erf(z / np.sqrt(2.0)))


def _grad_sign_slip(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + of.erf(z / np.sqrt(2.0))) - z * np.exp(-0.5 * z * z) / np.sqrt(2 * np.pi)


@pytest.mark.parametrize("slip", [_grad_missing_density, _grad_sign_slip],
                         ids=["no-density-term", "density-sign"])
def test_planted_gelu_grad_slip_is_caught(monkeypatch, slip):
    assert _pin_grad_table() and _pin_grads_autograd()
    monkeypatch.setattr(of, "gelu_grad", slip)
    assert not _pin_grad_table(of.gelu_grad)
    assert not _pin_grads_autograd()


def test_planted_weight_gradient_transposed_is_caught():
    def slipped(x, w1, w2, dout):
        dx, dw1, dw2 = feedforward_grads(x, w1, w2, dout)
        return dx, dw1, dw2.T.reshape(dw2.shape)   # dW2 laid out as [d_ff, d_model]
    assert not _pin_grads_autograd(slipped, d_model=12, d_ff=12)


def test_grad_rss_is_the_root_sum_square_of_the_term_sensitivities():
    """Entry by entry (scalar loops, math.fsum): the root-sum-square over the
    entry's terms of each term's sensitivity |dH| (2|GELU'| + |z GELU''|)
    |w1 or x| (dx, dW1) or |dOut| (|GELU| + |z GELU'|) (dW2), with GELU''
    the derivative of the printed-table-pinned GELU' taken by central
    differences; never below the largest term itself."""
    from oracle import feedforward_grad_rss
    rng = np.random.default_rng(14)
    x, w1, w2 = _rand(rng, 6, 4, 5)
    x[0, 0] = -0.75 * 2.0  # some pre-activations near GELU'(z) = 0
    dout = rng.standard_normal((6, 4))
    sdx, sdw1, sdw2 = feedforward_grad_rss(x, w1, w2, dout)
    z = x @ w1.T
    h = 1e-5
    def g2(v):
        return (float(gelu_grad(v + h)) - float(gelu_grad(v - h))) / (2 * h)
    dh = [[math.fsum(dout[r, c] * w2[c, f] for c in range(4)) for f in range(5)] for r in range(6)]
    sens = [[abs(dh[r][f]) * (2 * abs(float(gelu_grad(z[r, f]))) + abs(z[r, f] * g2(z[r, f])))
             for f in range(5)] for r in range(6)]
    hs = [[abs(float(gelu(z[r, f]))) + abs(z[r, f] * float(gelu_grad(z[r, f]))) for f in range(5)]
          for r in range(6)]
    cases = {
        "dx": (sdx, [[[sens[r][f] * abs(w1[f, c]) for f in range(5)] for c in range(4)] for r in range(6)]),
        "dw1": (sdw1, [[[sens[r][f] * abs(x[r, c]) for r in range(6)] for c in range(4)] for f in range(5)]),
        "dw2": (sdw2, [[[abs(dout[r, c]) * hs[r][f] for r in range(6)] for f in range(5)] for c in range(4)]),
    }
    dx, dw1, dw2 = feedforward_grads(x, w1, w2, dout)
    terms_max = {"dx": np.abs(dx), "dw1": np.abs(dw1), "dw2": np.abs(dw2)}
    for name, (got, t) in cases.items():
        for i, row in enumerate(t):
            for j, ts in enumerate(row):
                want = math.sqrt(math.fsum(v * v for v in ts))
                assert abs(got[i, j] - want) <= 1e-7 * max(1.0, want), (name, i, j)
    # each term's sensitivity is at least its magnitude, so the scale is at
    # least |g| / sqrt(number of terms)
    for name, n in (("dx", 5), ("dw1", 6), ("dw2", 6)):
        assert (cases[name][0] * np.sqrt(n) + 1e-12 >= terms_max[name]).all()


def test_rss_gate_passes_bf16_rounding_and_catches_a_one_row_slip():
    """The feedforward-gradient gate, |g - ref| <= 1e-2 scale + floor, on the
    CPU: gradients formed the way the kernels form them (bf16 operands, bf16
    Z, dH, dZ and H, fp32 products) pass it, for many rows and for one, while
    the same gradients with one row of dW1 off by 5 % of rms(dW1) fail it (a
    slip that the relative Frobenius guard alone does not see)."""
    import torch
    from oracle import feedforward_grad_rss
    from tests._gates import check_rss
    rng = np.random.default_rng(3)
    rows, dm, dff = 384, 128, 256
    def bf(a):
        return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()
    x = bf(rng.standard_normal((rows, dm)))
    w1 = bf(rng.standard_normal((dff, dm)) / np.sqrt(dm))
    w2 = bf(rng.standard_normal((dm, dff)) / np.sqrt(dff))
    dout = bf(rng.standard_normal((rows, dm)))
    zb = bf((x @ w1.T).astype(np.float32))
    dzb = bf(bf((dout @ w2).astype(np.float32)) * gelu_grad(zb))
    hb = bf(gelu(zb))
    got = [(dzb @ w1).astype(np.float32), (dzb.T @ x).astype(np.float32),
           (dout.T @ hb).astype(np.float32)]
    ref = feedforward_grads(x, w1, w2, dout)
    rss = feedforward_grad_rss(x, w1, w2, dout)
    for name, g, r, q in zip(("dx", "dw1", "dw2"), got, ref, rss):
        check_rss(name, g, r, q)
    one = slice(0, 1)
    r1 = feedforward_grads(x[one], w1, w2, dout[one])
    q1 = feedforward_grad_rss(x[one], w1, w2, dout[one])
    g1 = [(dzb[one] @ w1).astype(np.float32), (dzb[one].T @ x[one]).astype(np.float32),
          (dout[one].T @ hb[one]).astype(np.float32)]
    for name, g, r, q in zip(("dx", "dw1", "dw2"), g1, r1, q1):
        check_rss(name + " one row", g, r, q)
    slipped = got[1].copy()
    slipped[7] += 0.05 * np.sqrt((ref[1] ** 2).mean())
    rel_f = np.linalg.norm(slipped - ref[1]) / np.linalg.norm(ref[1])
    assert rel_f < 1e-2, "the slip must be invisible to the Frobenius guard"
    with pytest.raises(AssertionError):
        check_rss("dw1", slipped, ref[1], rss[1])
