"""Debug switches of the ring share on the GPU, through the C ABI.

* RA_NO_SKIP: the causal diagonal block computes every tile (those wholly
  above the diagonal fully masked) instead of skipping them; the results are
  bitwise those of the skipping path, forward and backward.
* The emulator's unsafe mode recycles a receive slot without waiting for the
  step that reads it and poisons it first: a negative control showing that
  the share's results, and so the parity gates, see the race the events
  prevent.  (Every access stays inside the caller's buffers; only values are
  wrong.)"""
import pytest
import torch

from blockwise_ring_attention_amd import share
from blockwise_ring_attention_amd.configs import ShareConfig

pytestmark = pytest.mark.gpu


def _share(host, **kw):
    dev = share.upload(host)
    share.forward(dev, **kw)
    share.backward(dev, **kw)
    torch.cuda.synchronize()
    return dev


NO_SKIP = [
    # (name, H, kv_heads, d, N, L, rank): the diagonal block is always seen
    ("d128 ragged", 2, 0, 128, 3, 300, 2),
    ("d64", 2, 0, 64, 2, 256, 1),
    ("gqa side by side", 4, 2, 128, 2, 200, 1),
    ("d128 2048 tokens", 8, 0, 128, 2, 2048, 1),
]


@pytest.mark.parametrize("case", NO_SKIP, ids=[c[0] for c in NO_SKIP])
def test_no_skip_is_bitwise(case, monkeypatch):
    name, H, hkv, d, N, L, rank = case
    print(name, flush=True)
    cfg = ShareConfig(90, name, "bf16", 1, H, d, N, L, (rank,), True, 256, 64,
                      backward=True, kv_heads=hkv)
    host = share.make_host_share(cfg, rank, seed=13, backward=True)
    monkeypatch.delenv("RA_NO_SKIP", raising=False)
    a = _share(host)
    monkeypatch.setenv("RA_NO_SKIP", "1")
    b = _share(host)
    monkeypatch.delenv("RA_NO_SKIP")
    for x, y, what in ((a.o_acc, b.o_acc, "o"), (a.lse_acc, b.lse_acc, "lse"),
                       (a.dq_acc, b.dq_acc, "dq")):
        assert torch.isfinite(x).all(), what
        assert torch.equal(x, y), what
    for kb, (x, y) in enumerate(zip(a.dkv_pool, b.dkv_pool)):
        if x is not None:
            assert torch.equal(x, y), f"dkv[{kb}]"


def test_no_skip_is_bitwise_fp32_forward(monkeypatch):
    """The fp32 forward (one query row per thread) under RA_NO_SKIP."""
    cfg = ShareConfig(92, "fp32 no-skip", "fp32", 1, 2, 64, 3, 200, (2,), True, 64, 64)
    host = share.make_host_share(cfg, 2, seed=14)
    outs = []
    for flag in (None, "1"):
        if flag is None:
            monkeypatch.delenv("RA_NO_SKIP", raising=False)
        else:
            monkeypatch.setenv("RA_NO_SKIP", flag)
        dev = share.upload(host)
        share.forward(dev)
        torch.cuda.synchronize()
        outs.append((dev.o_acc.clone(), dev.lse_acc.clone()))
    monkeypatch.delenv("RA_NO_SKIP")
    assert torch.isfinite(outs[0][0]).all()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def _rel(x, ref):
    return (torch.linalg.vector_norm(x - ref) / torch.linalg.vector_norm(ref)).item()


def test_unsafe_emulator_mode_is_seen():
    """Training share of 8192 tokens per member (rank 3 of 4, 32 heads): each
    step runs for milliseconds while a hop takes about 0.1 ms, so without the
    consume wait a slot is recycled (poisoned, then overwritten by a later
    block) before the step that reads it has run.  The safe run matches the
    oracle elsewhere; the unsafe one must be far from it."""
    cfg = ShareConfig(91, "unsafe", "bf16", 1, 32, 128, 4, 8192, (3,), True, 256, 64,
                      backward=True)
    host = share.make_host_share(cfg, 3, seed=3, backward=True)
    safe = _share(host)
    bad = _share(host, unsafe=True)

    def caught(x, ref):
        return not torch.isfinite(x).all().item() or _rel(x, ref) > 1e-2

    assert caught(bad.o_acc, safe.o_acc)
    assert caught(bad.dq_acc, safe.dq_acc)
    assert any(caught(x, y) for x, y in zip(bad.dkv_pool, safe.dkv_pool) if x is not None)
