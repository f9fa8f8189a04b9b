"""The blockwise feedforward, written out plainly in float64.

Test infrastructure only (see the package docstring).

Ring Attention with Blockwise Transformers (abstract) computes self-attention
and the feedforward blockwise; the sourcepulse project page (How It Works)
says both are distributed across devices.  Neither page gives the
feedforward's form.  Reading used: the position-wise two-layer MLP of a
transformer layer,

    FFN(x) = GELU(x W1^T) W2^T,     GELU(z) = z Phi(z) = z/2 (1 + erf(z/sqrt 2)),

applied to every row of x independently, with W1 [d_ff, d_model] and W2
[d_model, d_ff] in the (out, in) layout of a linear layer.  Because it is
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
