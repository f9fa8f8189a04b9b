"""Plain fp64 CPU oracle for one ring member's share of exact attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from here.  The
product path (the HIP library and its Python binding) never imports, calls or
falls back to this package, and this package imports nothing from the product
path: the two share no code.

What it computes
----------------
* ``attention``: the plain definition of softmax attention with a causal mask
  over global token positions, O = softmax(scale * Q K^T + M) V, plus the
  natural-log log-sum-exp of every query row.  Ring attention is exact (Ring
  Attention keyword page, definition: no approximation is involved;
  Ring Attention with Blockwise Transformers, abstract), so the share of a
  ring member equals this definition restricted to the member's rows.
* ``attention_grads``: the closed-form exact gradient of sum(dO * O).
* ``attention_grads_at_keys``: the same dK / dV restricted to chosen keys,
  for shares too long to hold dS whole.
* ``ffn.feedforward``: the position-wise two-layer MLP GELU(x W1^T) W2^T
  that the blockwise feedforward computes chunk by chunk (Ring Attention
  with Blockwise Transformers, abstract: attention and the feedforward are
  both computed block by block; the form is a reading, the pages give none).
* ``ffn.feedforward_grads``: its closed-form gradient (dx, dW1, dW2).
* ``brute``: scalar triple loops with ``math.exp`` / ``math.fsum`` for tiny
  shapes.
* ``ring``: a separate fp64 emulation of the ring schedule, the chunked online
  softmax and the associative combine (darcstar research page, commentary on
  online softmax being associative and on exact seams).  It exists to check
  ring-size, chunk-size and arrival-order invariance against ``attention``.

Pins (see ``tests/test_oracle_*.py``): brute force, closed forms stored under
``tests/golden/``, softmax rows summing to one, causal independence, key-shift
and value-linearity identities, finite differences for the gradients, torch
fp64 autograd and SDPA as independent library routines, gradient sum
identities, combine associativity / commutativity / identity.
"""
from .exact import attention, attention_grads, attention_grads_at_keys, positions
from .ffn import feedforward, feedforward_grad_rss, feedforward_grads, gelu, gelu_grad
from .ring import combine, block_partial, ring_share, ring_schedule

__all__ = ["attention", "attention_grads", "attention_grads_at_keys", "positions", "combine",
           "block_partial", "ring_share", "ring_schedule", "feedforward", "feedforward_grads",
           "feedforward_grad_rss", "gelu", "gelu_grad"]
