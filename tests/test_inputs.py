"""The seeded input generators (blockwise_ring_attention_amd/inputs.py): the
oracle and the GPU path consume exactly these tensors, so they must be
deterministic, independent per (config, tensor, block), of the stated
distributions and shapes, and rounded to bf16 from their float32 draw."""
import numpy as np
import torch

from blockwise_ring_attention_amd.configs import DecodeConfig, Dist, FfnConfig, ShareConfig
from blockwise_ring_attention_amd.inputs import (draw, draw_decode, draw_ffn, draw_ffn_dout,
                                                 draw_kv)

CFG = ShareConfig(80, "inputs", "bf16", batch=2, heads=4, head_dim=64, ring_size=4,
                  block_len=96, ranks=(1,), causal=True, q_chunk=64, k_chunk=64, kv_heads=2,
                  dists={"v": Dist("uniform", 1.0), "k": Dist("normal", 3.0)})


def test_deterministic_and_independent_streams():
    a = draw(CFG, "q", 2, seed=0)
    assert torch.equal(a, draw(CFG, "q", 2, seed=0))
    assert not torch.equal(a, draw(CFG, "q", 3, seed=0))      # another block
    assert not torch.equal(a, draw(CFG, "q", 2, seed=1))      # another seed
    assert not torch.equal(a, draw(CFG, "do", 2, seed=0))     # another tensor
    # a block's data does not depend on which member or length asks first
    b = draw(CFG, "q", 2, seed=0, length=40)
    assert torch.equal(b, draw(CFG, "q", 2, seed=0, length=40))


def test_shapes_dtypes_and_shared_heads():
    q = draw(CFG, "q", 0)
    kv = draw_kv(CFG, 0)
    assert q.shape == (2, 4, 96, 64) and q.dtype == torch.bfloat16
    assert kv.shape == (2, 2, 2, 96, 64) and kv.dtype == torch.bfloat16
    assert torch.equal(kv[0], draw(CFG, "k", 0)) and torch.equal(kv[1], draw(CFG, "v", 0))
    fp32 = ShareConfig(81, "fp32", "fp32", 1, 2, 64, 2, 32, (0,), True, 64, 64)
    assert draw(fp32, "q", 0).dtype == torch.float32


def test_distributions():
    big = ShareConfig(82, "dist", "fp32", 4, 8, 128, 2, 512, (0,), True, 64, 64,
                      dists={"k": Dist("normal", 3.0), "v": Dist("uniform", 1.0)})
    q, k, v = (draw(big, t, 0).double() for t in ("q", "k", "v"))
    assert abs(q.mean().item()) < 0.01 and abs(q.std().item() - 1.0) < 0.01
    assert abs(k.std().item() - 3.0) < 0.03
    assert v.min().item() >= -1.0 and v.max().item() < 1.0
    assert abs(v.std().item() - 1 / np.sqrt(3.0)) < 0.01


def test_bf16_is_the_rounded_float32_draw():
    f32 = ShareConfig(80, "inputs", "fp32", batch=2, heads=4, head_dim=64, ring_size=4,
                      block_len=96, ranks=(1,), causal=True, q_chunk=64, k_chunk=64)
    b16 = ShareConfig(80, "inputs", "bf16", batch=2, heads=4, head_dim=64, ring_size=4,
                      block_len=96, ranks=(1,), causal=True, q_chunk=64, k_chunk=64)
    x = draw(f32, "q", 1)
    assert torch.equal(draw(b16, "q", 1), x.to(torch.bfloat16))


def test_decode_and_feedforward_generators():
    cfg = DecodeConfig(83, "dec", 2, 8, 128, 3, 100, blocks=2, kv_heads=2)
    q, kvs = draw_decode(cfg, seed=4)
    assert q.shape == (2, 8, 3, 128) and len(kvs) == 2
    assert all(kv.shape == (2, 2, 2, 100, 128) for kv in kvs)
    assert not torch.equal(kvs[0], kvs[1])
    f = FfnConfig(84, "ffn", rows=300, d_model=256, d_ff=1024, chunk_rows=128)
    x, w1, w2 = draw_ffn(f, seed=2)
    dout = draw_ffn_dout(f, seed=2)
    assert x.shape == (300, 256) and w1.shape == (1024, 256) and w2.shape == (256, 1024)
    assert dout.shape == (300, 256) and dout.dtype == torch.bfloat16
    assert abs(w1.double().std().item() - 256 ** -0.5) < 0.003
    assert abs(w2.double().std().item() - 1024 ** -0.5) < 0.0015
    assert not torch.equal(x, dout)
    x2, _, _ = draw_ffn(f, seed=2)
    assert torch.equal(x, x2)
