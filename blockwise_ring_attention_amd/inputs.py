"""Seeded synthetic inputs for a ring member's share.

This module only draws random numbers; it holds no attention arithmetic.  The
oracle and the GPU path both consume exactly the host tensors it returns.

Each (config, tensor, global block) has its own NumPy stream, so the data of
a global block does not depend on which member looks at it, and no code path
ever needs to build the whole sequence in one place.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import DecodeConfig, FfnConfig, ShareConfig

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3, "x": 4, "w1": 5, "w2": 6}


def _rng(seed: int, cfg_id: int, tensor: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(cfg_id, TENSOR_ID[tensor], block))
    return np.random.default_rng(ss)


def draw(cfg: ShareConfig | DecodeConfig, tensor: str, block: int, seed: int = 0,
         length: int | None = None) -> torch.Tensor:
    """One [B, heads, length, d] block of ``tensor`` in the config's dtype
    (CPU); keys and values have the config's key/value head count.

    Values are drawn in float32 and rounded to bf16 with round-to-nearest-even
    for bf16 configs, so both consumers see identical rounded inputs."""
    L = cfg.block_len if length is None else length
    heads = cfg.n_kv_heads if tensor in ("k", "v") else cfg.heads
    shape = (cfg.batch, heads, L, cfg.head_dim)
    dist = cfg.dist(tensor)
    g = _rng(seed, cfg.cfg_id, tensor, block)
    if dist.kind == "normal":
        x = g.standard_normal(shape, dtype=np.float32)
        if dist.scale != 1.0:
            x *= np.float32(dist.scale)
    elif dist.kind == "uniform":
        x = g.random(shape, dtype=np.float32)
        x *= np.float32(2.0 * dist.scale)
        x -= np.float32(dist.scale)
    else:
        raise ValueError(f"unknown distribution {dist.kind!r}")
    t = torch.from_numpy(x)
    if cfg.dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif cfg.dtype != "fp32":
        raise ValueError(f"unknown dtype {cfg.dtype!r}")
    return t


def draw_kv(cfg: ShareConfig | DecodeConfig, block: int, seed: int = 0) -> torch.Tensor:
    """Packed key/value block [2, B, Hkv, L, d]: index 0 = K, 1 = V."""
    k = draw(cfg, "k", block, seed)
    v = draw(cfg, "v", block, seed)
    return torch.stack([k, v], dim=0)


def draw_decode(cfg: DecodeConfig, seed: int = 0):
    """Inputs of a decode-shaped share: query rows [B, H, Lq, d] (drawn as
    block ``cfg.blocks``, the one after every key) and the ``cfg.blocks``
    packed key/value blocks [2, B, Hkv, Lk, d], in arrival order."""
    q = draw(cfg, "q", cfg.blocks, seed, length=cfg.q_len)
    return q, [draw_kv(cfg, i, seed) for i in range(cfg.blocks)]


def draw_ffn(cfg: FfnConfig, seed: int = 0):
    """Inputs of the blockwise feedforward, bf16 (RNE from float32):
    x [rows, d_model] ~ N(0, 1), w1 [d_ff, d_model] ~ N(0, 1/d_model),
    w2 [d_model, d_ff] ~ N(0, 1/d_ff)."""
    out = []
    for name, shape, std in (("x", (cfg.rows, cfg.d_model), 1.0),
                             ("w1", (cfg.d_ff, cfg.d_model), cfg.d_model ** -0.5),
                             ("w2", (cfg.d_model, cfg.d_ff), cfg.d_ff ** -0.5)):
        a = _rng(seed, cfg.cfg_id, name, 0).standard_normal(shape, dtype=np.float32)
        a *= np.float32(std)
        out.append(torch.from_numpy(a).to(torch.bfloat16))
    return tuple(out)


def draw_ffn_dout(cfg: FfnConfig, seed: int = 0) -> torch.Tensor:
    """Upstream gradient of the feedforward's output, [rows, d_model] ~ N(0, 1),
    bf16 (RNE from float32)."""
    a = _rng(seed, cfg.cfg_id, "do", 0).standard_normal((cfg.rows, cfg.d_model),
                                                        dtype=np.float32)
    return torch.from_numpy(a).to(torch.bfloat16)


def torch_dtype(cfg: ShareConfig | DecodeConfig) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
