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
from blockwise_ring_attention_amd.inputs import draw_ffn, draw_ffn_dout
from tests._gates import check, check_rss

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


# ---- backward ----------------------------------------------------------------

def _run_bwd(x, w1, w2, dout, chunk, dw1=None, dw2=None):
    dev = torch.device("cuda:0")
    rows, d_model = x.shape
    d_ff = w1.shape[0]
    xd, w1d, w2d, dd = (t.to(dev) for t in (x, w1, w2, dout))
    dx = torch.empty((rows, d_model), dtype=torch.bfloat16, device=dev)
    dw1 = torch.zeros((d_ff, d_model), dtype=torch.float32, device=dev) if dw1 is None else dw1
    dw2 = torch.zeros((d_model, d_ff), dtype=torch.float32, device=dev) if dw2 is None else dw2
    nbytes = _lib.ring_ffn_bwd_workspace(rows, d_model, d_ff, chunk)
    work = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _lib.ring_ffn_bwd(xd, w1d, w2d, dd, dx, dw1, dw2, work, chunk)
    torch.cuda.synchronize()
    return dx.cpu(), dw1, dw2


BWD = [
    # (name, rows, d_model, d_ff, chunk_rows)
    ("one row", 1, 256, 256, 64),
    ("ragged rows, chunks off the tile grid", 300, 256, 512, 100),
    ("several tiles", 777, 512, 768, 512),
]


@pytest.mark.parametrize("case", BWD, ids=[c[0] for c in BWD])
def test_ffn_backward_small_elementwise(case):
    name, rows, dm, dff, chunk = case
    print(name, flush=True)
    cfg = FfnConfig(99, name, rows, dm, dff, chunk)
    x, w1, w2 = draw_ffn(cfg, seed=5)
    dout = draw_ffn_dout(cfg, seed=5)
    dx, dw1, dw2 = _run_bwd(x, w1, w2, dout, chunk)
    rdx, rdw1, rdw2 = oracle.feedforward_grads(x, w1, w2, dout)
    mdx, mdw1, mdw2 = oracle.feedforward_grad_rss(x, w1, w2, dout)
    check_rss("dx", dx, rdx, mdx)
    check_rss("dw1", dw1, rdw1, mdw1)
    check_rss("dw2", dw2, rdw2, mdw2)


def test_ffn_backward_accumulates_weight_gradients():
    """dw1 / dw2 gather contributions: two calls give twice the gradient, and
    dx does not depend on the chunking (bitwise)."""
    cfg = FfnConfig(99, "acc", 600, 256, 512, 0)
    x, w1, w2 = draw_ffn(cfg, seed=6)
    dout = draw_ffn_dout(cfg, seed=6)
    dx1, dw1, dw2 = _run_bwd(x, w1, w2, dout, 600)
    one1, one2 = dw1.clone(), dw2.clone()
    dx2, dw1, dw2 = _run_bwd(x, w1, w2, dout, 600, dw1, dw2)
    torch.testing.assert_close(dw1, 2 * one1, rtol=1e-6, atol=1e-6)
    torch.testing.assert_close(dw2, 2 * one2, rtol=1e-6, atol=1e-6)
    assert torch.equal(dx1, dx2)
    dx3, _, _ = _run_bwd(x, w1, w2, dout, 128)
    assert torch.equal(dx1, dx3)


def test_ffn_backward_full_size_sampled():
    """The benchmark's workload: dx on sampled rows; dW1 rows and dW2 columns
    of sampled hidden units (each hidden unit's weight gradients depend on
    that unit alone, so the oracle computes them on the reduced layer)."""
    cfg = FFN_CONFIGS["ffn-lwm7b"]
    print(cfg.name + " backward", flush=True)
    x, w1, w2 = draw_ffn(cfg, seed=0)
    dout = draw_ffn_dout(cfg, seed=0)
    dx, dw1, dw2 = _run_bwd(x, w1, w2, dout, cfg.chunk_rows)
    rng = np.random.default_rng(1)
    rows = np.array(sorted({0, 255, 256, cfg.chunk_rows - 1, cfg.chunk_rows, cfg.rows - 1}
                           | set(rng.choice(cfg.rows, size=12, replace=False).tolist())))
    rdx, _, _ = oracle.feedforward_grads(x[rows], w1, w2, dout[rows])
    mdx, _, _ = oracle.feedforward_grad_rss(x[rows], w1, w2, dout[rows])
    check_rss("dx", dx[rows], rdx, mdx)
    fs = np.array(sorted({0, 255, 256, cfg.d_ff - 1} |
                         set(rng.choice(cfg.d_ff, size=8, replace=False).tolist())))
    _, r1, r2 = oracle.feedforward_grads(x, w1[fs], w2[:, fs], dout)
    _, m1, m2 = oracle.feedforward_grad_rss(x, w1[fs], w2[:, fs], dout)
    sel = torch.from_numpy(fs).cuda()
    check_rss("dw1", dw1[sel].cpu(), r1, m1)
    check_rss("dw2", dw2[:, sel].cpu(), r2, m2)
