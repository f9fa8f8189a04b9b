"""The single-GPU ring emulator: overlap and serialize modes agree bitwise,
arrival order does not change the result beyond rounding, the state after a
partial ring equals the oracle on the blocks seen, and resuming from a saved
(o_acc, lse_acc) reproduces an uninterrupted run bitwise."""
import numpy as np
import pytest
import torch

import oracle
from blockwise_ring_attention_amd import _lib, share
from blockwise_ring_attention_amd.configs import ShareConfig
from tests._gates import check, check_lse

pytestmark = pytest.mark.gpu

CFG = ShareConfig(98, "emu", "bf16", 1, 4, 128, 6, 256, (4,), True, 256, 64)


@pytest.fixture(scope="module")
def host():
    return share.make_host_share(CFG, 4, seed=11)


def test_overlap_equals_serialize_bitwise(host):
    a = share.upload(host)
    share.forward(a, side_stream=torch.cuda.Stream())
    b = share.upload(host)
    share.forward(b, serialize=True)
    torch.cuda.synchronize()
    assert torch.equal(a.o_acc, b.o_acc) and torch.equal(a.lse_acc, b.lse_acc)


def test_arrival_order_invariance(host):
    ref = share.upload(host)
    share.forward(ref)
    rng = np.random.default_rng(0)
    for _ in range(3):
        order = rng.permutation(CFG.ring_size).tolist()
        dev = share.upload(host)
        share.forward(dev, order=order, side_stream=torch.cuda.Stream())
        torch.cuda.synchronize()
        np.testing.assert_allclose(dev.o_acc.cpu().numpy(), ref.o_acc.cpu().numpy(), atol=2e-6)
        np.testing.assert_allclose(dev.lse_acc.cpu().numpy(), ref.lse_acc.cpu().numpy(), atol=2e-6)


def test_partial_ring_state_and_resume(host):
    """After the first s steps the accumulators equal the definition on the
    blocks seen so far; saving them to the host and resuming the remaining
    steps reproduces the full run bitwise."""
    dev = share.upload(host)
    full = share.upload(host)
    share.forward(full)
    _lib.ring_attn_init_acc(dev.o_acc, dev.lse_acc)
    sched = oracle.ring_schedule(4, CFG.ring_size)
    stop = 3
    for s in range(stop):
        kb = sched[s]
        _lib.ring_attn_fwd(dev.q, dev.pool[kb] if dev.pool[kb] is not None else dev.slots[0], 4, s,
                           CFG.ring_size, True, 256, 64, dev.o_acc, dev.lse_acc)
    torch.cuda.synchronize()
    seen = [b for b in sched[:stop] if b <= 4]
    L = CFG.block_len
    k = torch.cat([host.kv[b][0] for b in seen], dim=2)
    v = torch.cat([host.kv[b][1] for b in seen], dim=2)
    kp = np.concatenate([oracle.positions(b, L) for b in seen])
    o_ref, lse_ref = oracle.attention(host.q, k, v, oracle.positions(4, L), kp, True)
    check("o after 3 steps", dev.o_acc, o_ref, "bf16")
    check_lse("lse after 3 steps", dev.lse_acc, lse_ref)
    # checkpoint: the whole resumable state is (o_acc, lse_acc)
    saved = (dev.o_acc.cpu(), dev.lse_acc.cpu())
    dev.o_acc.fill_(float("nan"))
    dev.lse_acc.fill_(0)
    dev.o_acc.copy_(saved[0])
    dev.lse_acc.copy_(saved[1])
    for s in range(stop, CFG.ring_size):
        kb = sched[s]
        if dev.pool[kb] is None:
            continue
        _lib.ring_attn_fwd(dev.q, dev.pool[kb], 4, s, CFG.ring_size, True, 256, 64,
                           dev.o_acc, dev.lse_acc)
    torch.cuda.synchronize()
    assert torch.equal(dev.o_acc, full.o_acc) and torch.equal(dev.lse_acc, full.lse_acc)


def test_only_two_receive_slots(host):
    """No all-gather: besides the member's own block and the pool that stands
    for the other members, the emulator touches exactly two slot buffers and
    allocates no device memory of its own."""
    dev = share.upload(host)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    share.forward(dev, side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert len(dev.slots) == 2


def test_back_to_back_shares_do_not_race():
    """Regression: a backward share enqueued right after the forward share
    (same receive slots, no host synchronisation) once overwrote slots the
    forward was still reading.  Short blocks make each compute step brief, so
    the hops of the next call would land during it.  Every result must equal
    the fully serialised run bitwise."""
    cfg = ShareConfig(99, "b2b", "bf16", 1, 4, 128, 4, 2048, (3,), True, 256, 64, backward=True)
    host = share.make_host_share(cfg, 3, backward=True)
    ref = share.upload(host)
    share.forward(ref, serialize=True)
    share.backward(ref, serialize=True)
    torch.cuda.synchronize()
    dev = share.upload(host)
    for _ in range(2):
        share.forward(dev)
        share.backward(dev)
    share.forward(dev)
    torch.cuda.synchronize()
    assert torch.equal(dev.o_acc, ref.o_acc) and torch.equal(dev.lse_acc, ref.lse_acc)
    assert torch.equal(dev.dq_acc, ref.dq_acc)
    for a, b in zip(dev.dkv_pool, ref.dkv_pool):
        assert torch.equal(a, 2 * b)          # two backward shares accumulated
