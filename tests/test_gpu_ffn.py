"""GPU parity of the blockwise feedforward (ring_ffn_fwd) against the fp64
oracle, through the C ABI.  Small cases are compared element by element
(several 256 x 256 tiles, ragged row tiles, chunks that are not multiples of
the tile); the full-size workload, in the chunking the benchmark uses, is
compared on sampled rows; chunking is checked to leave every row bitwise
unchanged."""
import numpy as np
import pytest
import torch

import oracle
from blockwise_ring_attention_amd import _lib
from blockwise_ring_attention_amd.configs import FFN_CONFIGS, FfnConfig
from blockwise_ring_attention_amd.inputs import draw_ffn
from tests._gates import check

pytestmark = pytest.mark.gpu


def _run(x, w1, w2, chunk):
    dev = torch.device("cuda:0")
    xd, w1d, w2d = x.to(dev), w1.to(dev), w2.to(dev)
    rows, d_model = x.shape
    hidden = torch.empty((min(rows, chunk), w1.shape[0]), dtype=torch.bfloat16, device=dev)
    out = torch.empty((rows, d_model), dtype=torch.bfloat16, device=dev)
    _lib.ring_ffn_fwd(xd, w1d, w2d, hidden, out, chunk)
    torch.cuda.synchronize()
    return out.cpu()


SMALL = [
    # (name, rows, d_model, d_ff, chunk_rows)
    ("one row", 1, 256, 256, 64),
    ("ragged rows, two chunks", 300, 256, 512, 256),
    ("chunks not a multiple of the tile", 777, 512, 1024, 300),
    ("several row tiles in one chunk", 1024, 256, 768, 4096),
    ("wide hidden", 257, 256, 2048, 257),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_ffn_small_elementwise(case):
    name, rows, dm, dff, chunk = case
    print(name, flush=True)
    x, w1, w2 = draw_ffn(FfnConfig(96, name, rows, dm, dff, chunk), seed=3)
    out = _run(x, w1, w2, chunk)
    check("out", out, oracle.feedforward(x, w1, w2), "bf16")


def test_ffn_chunking_leaves_rows_bitwise_unchanged():
    x, w1, w2 = draw_ffn(FfnConfig(97, "chunks", 700, 512, 1024, 0), seed=4)
    outs = [_run(x, w1, w2, c) for c in (700, 256, 100, 1)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_ffn_full_size_sampled_rows():
    """The benchmark's workload (16384 rows of width 4096 through a 16384-wide
    hidden layer, 4096 rows per chunk) on rows at chunk and tile seams plus
    random ones."""
    cfg = FFN_CONFIGS["ffn-lwm7b"]
    print(cfg.name, flush=True)
    x, w1, w2 = draw_ffn(cfg, seed=0)
    out = _run(x, w1, w2, cfg.chunk_rows)
    rng = np.random.default_rng(0)
    rows = {0, 1, 255, 256, cfg.rows - 1}
    for c in range(cfg.chunk_rows, cfg.rows, cfg.chunk_rows):
        rows.update({c - 1, c})
    rows.update(rng.choice(cfg.rows, size=24, replace=False).tolist())
    rows = np.array(sorted(rows))
    ref = oracle.feedforward(x[rows], w1, w2)
    check("out", out[rows], ref, "bf16")
