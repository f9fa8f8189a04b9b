"""The blockwise feedforward, written out plainly in float64.

Test infrastructure only (see the package docstring).

Ring Attention with Blockwise Transformers (abstract) computes self-attention
and the feedforward blockwise; the sourcepulse project page (How It Works)
says both are distributed across devices.  Neither page gives the
feedforward's form.  Reading used: the position-wise two-layer MLP of a
transformer layer,

    FFN(x) = GELU(x W1^T) W2^T,     GELU(z) = z Phi(z) = z/2 (1 + erf(z/sqrt 2)),

applied to every row of x independently, with W1 [d_ff, d_model] and W2
[d_model, d_ff] in the (out, in) layout of a linear layer.  The gradients
(the pages do not discuss the backward) are those of sum(dOut * FFN(x)):
with Z = x W1^T, H = GELU(Z), dH = dOut W2 and dZ = dH * GELU'(Z),
GELU'(z) = Phi(z) + z phi(z):  dx = dZ W1,  dW1 = dZ^T x,  dW2 = dOut^T H.  Because it is
position-wise, computing it a chunk of rows at a time (the blockwise form)
gives the same rows; the oracle therefore evaluates all rows at once, with
no rounding of the hidden activation.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


def _as64(x) -> np.ndarray:
    if hasattr(x, "detach"):          # torch tensor (bf16 has no numpy dtype)
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def gelu(z):
    """GELU with the Gaussian CDF in its exact (erf) form."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def feedforward(x, w1, w2):
    """FFN of every row of x [rows, d_model]: returns float64 [rows, d_model]."""
    x, w1, w2 = _as64(x), _as64(w1), _as64(w2)
    if w1.shape[1] != x.shape[1] or w2.shape != (w1.shape[1], w1.shape[0]):
        raise ValueError(f"shapes x {x.shape}, w1 {w1.shape}, w2 {w2.shape} do not chain")
    return gelu(x @ w1.T) @ w2.T


def gelu_grad(z):
    """d GELU / dz = Phi(z) + z phi(z), phi the standard normal density."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def feedforward_grads(x, w1, w2, dout):
    """Gradients of sum(dout * FFN(x)) with respect to x, W1 and W2, float64:
    returns (dx [rows, d_model], dw1 [d_ff, d_model], dw2 [d_model, d_ff])."""
    x, w1, w2, dout = _as64(x), _as64(w1), _as64(w2), _as64(dout)
    if w1.shape[1] != x.shape[1] or w2.shape != (w1.shape[1], w1.shape[0]):
        raise ValueError(f"shapes x {x.shape}, w1 {w1.shape}, w2 {w2.shape} do not chain")
    if dout.shape != x.shape:
        raise ValueError(f"dout {dout.shape} does not match x {x.shape}")
    z = x @ w1.T
    h = gelu(z)
    dz = (dout @ w2) * gelu_grad(z)
    return dz @ w1, dz.T @ x, dout.T @ h


def gelu_grad2(z):
    """d^2 GELU / dz^2 = phi(z) (2 - z^2)."""
    z = np.asarray(z, dtype=np.float64)
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi) * (2.0 - z * z)


def feedforward_grad_rss(x, w1, w2, dout):
    """Error scale of each gradient entry: the root-sum-square, over the terms
    behind the entry, of each term's first-order sensitivity to relative
    perturbations of the intermediates it is formed from (dH, Z and dZ for
    the terms dZ * W1 of dx and dZ * x of dW1, where dZ = dH GELU'(Z);
    Z and H = GELU(Z) for the terms dOut * H of dW2):
        dx, dW1:  |dH| (2 |GELU'(z)| + |z GELU''(z)|) times |W1| or |x|
        dW2:      |dOut| (|GELU(z)| + |z GELU'(z)|)
    Float64, same shapes as feedforward_grads.  If each intermediate carries
    an independent relative error of RMS e, an entry's error has RMS at most
    about e times this value, however much the terms cancel (and a term whose
    own value vanishes, GELU'(z) = 0, still has its sensitivity to z)."""
    x, w1, w2, dout = _as64(x), _as64(w1), _as64(w2), _as64(dout)
    z = x @ w1.T
    sens = np.abs(dout @ w2) * (2.0 * np.abs(gelu_grad(z)) + np.abs(z * gelu_grad2(z)))
    s2 = sens ** 2
    hs = np.abs(gelu(z)) + np.abs(z * gelu_grad(z))
    return (np.sqrt(s2 @ (w1 * w1)), np.sqrt(s2.T @ (x * x)),
            np.sqrt((dout * dout).T @ (hs * hs)))
