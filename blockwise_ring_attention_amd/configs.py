"""The five ring-member workloads, as plain data.

A ring of ``ring_size`` members splits one sequence into equal contiguous
blocks of ``block_len`` tokens; member r holds the queries of block r and sees
the key/value blocks as they circulate (Ring Attention definition on the
chapterpal "Ring Attention" keyword page; "Blockwise RingAttention" keyword
page, definition).  ``q_chunk`` / ``k_chunk`` are the query/key chunk sizes
that the sourcepulse project page lists as performance-tuning knobs
(Highlighted Details).  Nothing here computes attention.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple


@dataclass(frozen=True)
class Dist:
    """How one input tensor is drawn: ``normal`` (mean 0) or ``uniform`` on
    (-scale, scale); ``scale`` is the standard deviation for ``normal``."""
    kind: str = "normal"
    scale: float = 1.0


@dataclass(frozen=True)
class ShareConfig:
    cfg_id: int
    name: str
    dtype: str                  # "fp32" or "bf16": dtype of q, k, v, dO
    batch: int
    heads: int
    head_dim: int
    ring_size: int
    block_len: int              # tokens per ring member (Lq == Lk)
    ranks: Tuple[int, ...]      # members whose share is computed
    causal: bool
    q_chunk: int
    k_chunk: int
    dists: Dict[str, Dist] = field(default_factory=dict)
    backward: bool = False
    kv_heads: int = 0           # key/value heads shared by groups of query heads; 0: heads

    @property
    def n_kv_heads(self) -> int:
        return self.kv_heads or self.heads

    def dist(self, tensor: str) -> Dist:
        return self.dists.get(tensor, Dist())

    def kv_blocks_seen(self, rank: int) -> Tuple[int, ...]:
        """Global block ids whose keys a member's queries can attend to.

        Under the causal mask a member never needs a block that lies after
        its own; without it, every block of the ring contributes."""
        if self.causal:
            return tuple(range(rank + 1))
        return tuple(range(self.ring_size))

    def pairs(self, rank: int) -> int:
        """Unmasked (query, key) pairs of one member's share over all (b, h)."""
        L = self.block_len
        if self.causal:
            per_head = rank * L * L + L * (L + 1) // 2
        else:
            per_head = self.ring_size * L * L
        return per_head * self.batch * self.heads


CONFIGS: Dict[int, ShareConfig] = {
    1: ShareConfig(
        1, "tiny-exact-fp32", "fp32", batch=1, heads=4, head_dim=64,
        ring_size=4, block_len=256, ranks=(0, 1, 2, 3), causal=True,
        q_chunk=64, k_chunk=64),
    2: ShareConfig(
        2, "noncausal-bf16", "bf16", batch=2, heads=16, head_dim=128,
        ring_size=8, block_len=4096, ranks=(0,), causal=False,
        q_chunk=512, k_chunk=1024),
    3: ShareConfig(
        3, "lwm7b-causal-fwd", "bf16", batch=1, heads=32, head_dim=128,
        ring_size=8, block_len=16384, ranks=(7,), causal=True,
        q_chunk=256, k_chunk=64,
        dists={"q": Dist("normal", 0.5), "k": Dist("normal", 0.5),
               "v": Dist("normal", 0.5)}),
    4: ShareConfig(
        4, "train-causal-fwd-bwd", "bf16", batch=1, heads=32, head_dim=128,
        ring_size=4, block_len=8192, ranks=(3,), causal=True,
        q_chunk=256, k_chunk=64, backward=True),
    5: ShareConfig(
        5, "million-token-adversarial", "bf16", batch=1, heads=32,
        head_dim=128, ring_size=64, block_len=16384, ranks=(31,),
        causal=True, q_chunk=256, k_chunk=64,
        dists={"q": Dist("normal", 3.0), "k": Dist("normal", 3.0),
               "v": Dist("uniform", 1.0)}),
}


@dataclass(frozen=True)
class DecodeConfig:
    """A decode-shaped share: ``q_len`` new query rows per (batch, head) that
    come after every key, attending to ``blocks`` key/value blocks of
    ``kv_len`` tokens folded one after another (a member's share of a long
    key/value cache, or the blocks that reach it around the ring).  The
    inference use of the method (Ring Attention with Blockwise Transformers,
    abstract).  ``k_chunk`` = 0 lets the library pick the key split."""
    cfg_id: int
    name: str
    batch: int
    heads: int
    head_dim: int
    q_len: int
    kv_len: int
    blocks: int = 1
    kv_heads: int = 0
    k_chunk: int = 0
    dtype: str = "bf16"
    scale: float = 0.0
    dists: Dict[str, Dist] = field(default_factory=dict)

    @property
    def n_kv_heads(self) -> int:
        return self.kv_heads or self.heads

    @property
    def block_len(self) -> int:   # default length of a drawn key/value block
        return self.kv_len

    def dist(self, tensor: str) -> Dist:
        return self.dists.get(tensor, Dist())


DECODE_CONFIGS: Dict[str, DecodeConfig] = {
    # One decode step of eight sequences for the 7B model's heads (32 x 128)
    # against one member's 16384-token share of the key/value cache.
    "decode-lwm7b": DecodeConfig(
        6, "decode-lwm7b", batch=8, heads=32, head_dim=128, q_len=1, kv_len=16384,
        dists={"q": Dist("normal", 0.5), "k": Dist("normal", 0.5),
               "v": Dist("normal", 0.5)}),
}


@dataclass(frozen=True)
class FfnConfig:
    """The blockwise feedforward of a member's rows: ``rows`` tokens of width
    ``d_model`` through a ``d_ff``-wide hidden layer, ``chunk_rows`` rows at a
    time (Ring Attention with Blockwise Transformers, abstract: blockwise
    feedforward).  x ~ N(0, 1); W1 ~ N(0, 1/d_model) and W2 ~ N(0, 1/d_ff),
    so pre-activations and outputs are of order one."""
    cfg_id: int
    name: str
    rows: int
    d_model: int
    d_ff: int
    chunk_rows: int


FFN_CONFIGS: Dict[str, FfnConfig] = {
    # One member's 16384-token block of the 7B model (width 32 x 128 = 4096,
    # hidden 4 x 4096), 4096 rows per chunk.
    "ffn-lwm7b": FfnConfig(7, "ffn-lwm7b", rows=16384, d_model=4096, d_ff=16384,
                           chunk_rows=4096),
}


def scaled(cfg: ShareConfig, **changes) -> ShareConfig:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    from dataclasses import replace
    return replace(cfg, **changes)
