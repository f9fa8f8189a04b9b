"""GPU parity of the backward ring share (dQ, and dK/dV per block in ring
order) against the oracle's closed-form gradients, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from blockwise_ring_attention_amd import _lib, share
from blockwise_ring_attention_amd.configs import CONFIGS, ShareConfig
from tests._gates import check, seam_rows, tile_rows

pytestmark = pytest.mark.gpu


def _oracle_grads(host, heads=None, rows=None, kv_head=None):
    """Oracle dQ and per-block dK/dV: every head (default), the given query
    heads of a multi-head share, or the query heads of one shared key/value
    head (kv_head)."""
    cfg = host.cfg
    L = cfg.block_len
    blocks = sorted(host.kv)
    if kv_head is not None:
        G = cfg.heads // host.kv[blocks[0]].shape[2]
        hs, ks = list(range(kv_head * G, (kv_head + 1) * G)), [kv_head]
    elif heads is None:
        hs, ks = list(range(cfg.heads)), list(range(host.kv[blocks[0]].shape[2]))
    else:
        hs = ks = heads
    k = torch.cat([host.kv[b][0][:, ks] for b in blocks], dim=2)
    v = torch.cat([host.kv[b][1][:, ks] for b in blocks], dim=2)
    q = host.q[:, hs]
    do = host.dout[:, hs]
    q_pos = oracle.positions(host.rank, L)
    if rows is not None:
        q, do, q_pos = q[:, :, rows], do[:, :, rows], q_pos[rows]
    k_pos = np.concatenate([oracle.positions(b, L) for b in blocks])
    dq, dk, dv, o, lse = oracle.attention_grads(q, k, v, do, q_pos, k_pos, cfg.causal)
    per_block = {b: (dk[:, :, i * L:(i + 1) * L], dv[:, :, i * L:(i + 1) * L])
                 for i, b in enumerate(blocks)}
    return dq, per_block


def _run(host, **kw):
    dev = share.upload(host)
    share.forward(dev, **kw)
    share.backward(dev, **kw)
    torch.cuda.synchronize()
    return dev


SMALL = [
    # (name, B, H, d, N, L, rank, causal)
    ("d128 causal ragged", 1, 2, 128, 3, 200, 2, True),
    ("d128 causal diagonal only", 1, 2, 128, 2, 256, 0, True),
    ("d64 causal", 1, 2, 64, 4, 96, 3, True),
    ("d128 noncausal", 2, 1, 128, 3, 160, 1, False),
    # degenerate lengths: one token per block, one row past a 32-row tile
    ("d128 causal single token", 1, 2, 128, 3, 1, 2, True),
    ("d128 causal 33 tokens", 1, 2, 128, 2, 33, 1, True),
    ("d64 noncausal 65 tokens", 1, 1, 64, 2, 65, 0, False),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_backward_elementwise(case):
    name, B, H, d, N, L, rank, causal = case
    print(name, flush=True)
    cfg = ShareConfig(95, name, "bf16", B, H, d, N, L, (rank,), causal, 256, 64, backward=True)
    host = share.make_host_share(cfg, rank, seed=7, backward=True)
    dev = _run(host)
    dq_ref, per_block = _oracle_grads(host)
    check("dq", dev.dq_acc, dq_ref, "bf16")
    for b, (dk_ref, dv_ref) in per_block.items():
        check(f"dk[{b}]", dev.dkv_pool[b][0], dk_ref, "bf16")
        check(f"dv[{b}]", dev.dkv_pool[b][1], dv_ref, "bf16")
    for b in range(N):
        if b not in per_block and dev.dkv_pool[b] is not None:
            assert (dev.dkv_pool[b] == 0).all()


def test_backward_is_deterministic_and_serialize_matches_overlap():
    cfg = ShareConfig(96, "det", "bf16", 1, 2, 128, 4, 192, (3,), True, 256, 64, backward=True)
    host = share.make_host_share(cfg, 3, backward=True)
    side = torch.cuda.Stream()
    a = _run(host, side_stream=side)
    b = share.upload(host)
    share.forward(b, serialize=True)
    share.backward(b, serialize=True)
    torch.cuda.synchronize()
    assert torch.equal(a.dq_acc, b.dq_acc)
    for x, y in zip(a.dkv_pool, b.dkv_pool):
        assert torch.equal(x, y)


def test_travelling_partial_accumulates():
    """dkv_io is +=: a partial that arrives non-zero keeps its contents."""
    cfg = ShareConfig(97, "acc", "bf16", 1, 1, 128, 2, 128, (1,), True, 256, 64, backward=True)
    host = share.make_host_share(cfg, 1, backward=True)
    dev = share.upload(host)
    share.forward(dev)
    base = [t.clone().normal_() for t in dev.dkv_pool]
    for t, s in zip(dev.dkv_pool, base):
        t.copy_(s)
    share.backward(dev, side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    _, per_block = _oracle_grads(host)
    for kb, (dk_ref, dv_ref) in per_block.items():
        got = dev.dkv_pool[kb] - base[kb]
        check(f"dk[{kb}]", got[0], dk_ref, "bf16")
        check(f"dv[{kb}]", got[1], dv_ref, "bf16")


def _dq_every_tile(host, dev, rng, seams):
    """dQ against the oracle on one random row of every 256-row query tile
    of every head (plus the seam rows): every workgroup of the dQ launches
    has a row checked."""
    cfg = host.cfg
    got, want = [], []
    for h in range(cfg.heads):
        rows = tile_rows(cfg.block_len, 256, rng, seams)
        dq_ref, _ = _oracle_grads(host, heads=[h], rows=rows)
        got.append(dev.dq_acc[:, [h]][:, :, rows].cpu())
        want.append(dq_ref)
    check("dq", torch.cat(got, dim=2), np.concatenate(want, axis=2), "bf16")


def test_cfg4_full_size():
    """Training share at full size: dQ on one row of every query tile of
    every head (plus seams), dK/dV of every block on two sampled heads
    (their gradients need every row)."""
    cfg = CONFIGS[4]
    rank = cfg.ranks[0]
    print("cfg4: generating inputs", flush=True)
    host = share.make_host_share(cfg, rank, backward=True)
    print("cfg4: running forward + backward share", flush=True)
    dev = _run(host, side_stream=torch.cuda.Stream())
    rng = np.random.default_rng(4)
    print(f"cfg4: oracle dq on every tile of {cfg.heads} heads", flush=True)
    _dq_every_tile(host, dev, rng, seam_rows(cfg.block_len, cfg.q_chunk, rng, 0))
    heads = sorted(rng.choice(cfg.heads, size=2, replace=False).tolist())
    for h in heads:
        print(f"cfg4: oracle dk/dv head {h}", flush=True)
        _, per_block = _oracle_grads(host, heads=[h])
        for kb, (dk_ref, dv_ref) in per_block.items():
            check(f"dk[{kb}] h{h}", dev.dkv_pool[kb][0][:, [h]], dk_ref, "bf16")
            check(f"dv[{kb}] h{h}", dev.dkv_pool[kb][1][:, [h]], dv_ref, "bf16")
    assert torch.isfinite(dev.dq_acc).all()


def test_causal_independence_bitwise():
    """Keys after position p (values too) never reach the rows at or before p:
    perturbing them leaves those rows of o, lse and dQ bitwise unchanged
    (the exact causal mask across seams; darcstar commentary)."""
    cfg = ShareConfig(96, "indep", "bf16", 1, 2, 128, 2, 300, (1,), True, 256, 64,
                      backward=True)
    host = share.make_host_share(cfg, 1, seed=11, backward=True)
    p = 137  # local position inside the diagonal block (a ragged, mid-tile row)
    g = torch.Generator().manual_seed(5)
    kv = host.kv[1].clone()
    kv[:, :, :, p + 1:] = (torch.randn(kv[:, :, :, p + 1:].shape, generator=g) * 2).to(kv.dtype)
    other = share.HostShare(cfg, 1, host.q, {0: host.kv[0], 1: kv}, host.dout)
    a, b = _run(host), _run(other)
    assert not torch.equal(a.o_acc[:, :, p + 1:], b.o_acc[:, :, p + 1:])  # the change matters
    assert torch.equal(a.o_acc[:, :, :p + 1], b.o_acc[:, :, :p + 1])
    assert torch.equal(a.lse_acc[:, :, :p + 1], b.lse_acc[:, :, :p + 1])
    assert torch.equal(a.dq_acc[:, :, :p + 1], b.dq_acc[:, :, :p + 1])


@pytest.mark.parametrize("use_work", [True, False], ids=["side-by-side", "one-by-one"])
@pytest.mark.parametrize("kv_heads", [1, 2])
def test_shared_kv_heads_backward(kv_heads, use_work):
    """MQA (one key/value head) and GQA (two, for four query heads): dK/dV of
    a shared head sums its query heads' contributions, element by element
    against the oracle, with the group's query heads side by side (4 for
    MQA, 2 for GQA here: 3 and 1 dK/dV copies in the workspace) or one
    launch per member."""
    cfg = ShareConfig(98, f"shared-kv{kv_heads}", "bf16", 1, 4, 128, 3, 200, (2,), True,
                      256, 64, backward=True, kv_heads=kv_heads)
    host = share.make_host_share(cfg, 2, seed=8, backward=True)
    assert host.kv[0].shape[2] == kv_heads
    dev = share.upload(host)
    assert (dev.work is not None) and dev.work.numel() == (4 // kv_heads - 1) * 2 * kv_heads * 200 * 128 * 4
    share.forward(dev)
    share.backward(dev, use_work=use_work)
    torch.cuda.synchronize()
    dq_ref, per_block = _oracle_grads(host)
    check("dq", dev.dq_acc, dq_ref, "bf16")
    for b, (dk_ref, dv_ref) in per_block.items():
        check(f"dk[{b}]", dev.dkv_pool[b][0], dk_ref, "bf16")
        check(f"dv[{b}]", dev.dkv_pool[b][1], dv_ref, "bf16")


def test_shared_kv_heads_full_size():
    """LWM-7B-shaped training share with eight key/value heads for 32 query
    heads (rank 3 of 4, 8192 tokens per member): dQ on sampled rows, dK/dV
    of one shared head against its four query heads' full rows."""
    cfg = ShareConfig(99, "gqa-train", "bf16", 1, 32, 128, 4, 8192, (3,), True, 256, 64,
                      backward=True, kv_heads=8)
    print("gqa: generating inputs", flush=True)
    host = share.make_host_share(cfg, 3, backward=True)
    print("gqa: running forward + backward share", flush=True)
    dev = _run(host)
    rng = np.random.default_rng(9)
    rows = seam_rows(cfg.block_len, cfg.q_chunk, rng, 12)
    heads = sorted(rng.choice(cfg.heads, size=3, replace=False).tolist())
    print(f"gqa: oracle dq on {len(rows)} rows of heads {heads}", flush=True)
    for h in heads:
        dq_ref, _ = _oracle_grads(host, kv_head=h // 4, rows=rows)
        check(f"dq h{h}", dev.dq_acc[:, [h]][:, :, rows], dq_ref[:, [h % 4]], "bf16")
    kh = int(rng.integers(8))
    print(f"gqa: oracle dk/dv of key/value head {kh}", flush=True)
    _, per_block = _oracle_grads(host, kv_head=kh)
    for kb, (dk_ref, dv_ref) in per_block.items():
        check(f"dk[{kb}] kvh{kh}", dev.dkv_pool[kb][0][:, [kh]], dk_ref, "bf16")
        check(f"dv[{kb}] kvh{kh}", dev.dkv_pool[kb][1][:, [kh]], dv_ref, "bf16")
    assert torch.isfinite(dev.dq_acc).all()


def test_mqa_full_size_side_by_side():
    """MQA share, 32 query heads on one key/value head (rank 3 of 4, 2048
    tokens per member): 16 query heads run side by side in two launches (15
    workspace copies stored by the first, added to by the second); dK/dV of
    every block and dQ of every head in full, against the oracle."""
    cfg = ShareConfig(99, "mqa-train", "bf16", 1, 32, 128, 4, 2048, (3,), True, 256, 64,
                      backward=True, kv_heads=1)
    host = share.make_host_share(cfg, 3, seed=5, backward=True)
    dev = share.upload(host)
    assert dev.work.numel() == 15 * 2 * 2048 * 128 * 4
    print("mqa: running forward + backward share", flush=True)
    share.forward(dev)
    share.backward(dev)
    torch.cuda.synchronize()
    print("mqa: oracle gradients of the whole share", flush=True)
    dq_ref, per_block = _oracle_grads(host)
    check("dq", dev.dq_acc, dq_ref, "bf16")
    for kb, (dk_ref, dv_ref) in per_block.items():
        check(f"dk[{kb}]", dev.dkv_pool[kb][0], dk_ref, "bf16")
        check(f"dv[{kb}]", dev.dkv_pool[kb][1], dv_ref, "bf16")


def test_mqa_benchmark_shape_side_by_side_matches_one_by_one():
    """The MQA training share at the benchmark's size (rank 7 of 8, 16384
    tokens per member, 32 query heads on one key/value head): two query
    heads side by side give dK/dV that differ from one head after another
    only by the order of fp32 additions, and are bitwise repeatable.  (Each
    dK/dV element sums all 32 heads' rows over 131072 keys: past what the
    oracle can take at this size; the sequential path is pinned to the
    oracle at full size for GQA.)"""
    cfg = ShareConfig(99, "mqa-bench", "bf16", 1, 32, 128, 8, 16384, (7,), True, 256, 64,
                      backward=True, kv_heads=1)
    host = share.make_host_share(cfg, 7, seed=0, backward=True)
    dev = share.upload(host)
    assert dev.work.numel() == 2 * 16384 * 128 * 4                      # one copy
    share.forward(dev)
    out = []
    for use_work in (True, True, False):
        print(f"mqa bench shape: backward use_work={use_work}", flush=True)
        for t in dev.dkv_pool:
            if t is not None:
                t.zero_()
        share.backward(dev, use_work=use_work)
        torch.cuda.synchronize()
        out.append(([t.clone() for t in dev.dkv_pool if t is not None], dev.dq_acc.clone()))
    (a, dqa), (b, dqb), (c, dqc) = out
    assert torch.equal(dqa, dqb) and torch.equal(dqa, dqc)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y)
        assert torch.isfinite(x).all()
        rel = (torch.linalg.vector_norm(x - z) / torch.linalg.vector_norm(z)).item()
        assert rel < 1e-5, rel
        assert (x - z).abs().max().item() <= 1e-4 * z.abs().max().item()


def test_benchmark_training_share_full_size():
    """The training share the benchmark times (rank 7 of a ring of 8, 16384
    tokens per member, 32 heads of 128, bf16, seed 0), run as the benchmark
    runs it (emulated ring with side-stream hops): dQ on one row of every
    query tile of every head; dK / dV of four heads at one key of every
    128-key tile (one dK/dV workgroup each) and at the tile seams of every
    block, whose gradients need every row of the share (the oracle takes
    each row's log-sum-exp and delta from a full pass, then only those key
    columns)."""
    from blockwise_ring_attention_amd.configs import scaled
    cfg = scaled(CONFIGS[3], backward=True)
    rank = cfg.ranks[0]
    L = cfg.block_len
    print("bench share: generating inputs", flush=True)
    host = share.make_host_share(cfg, rank, seed=0, backward=True)
    print("bench share: running forward + backward", flush=True)
    dev = _run(host, side_stream=share.side_stream_for(torch.device("cuda:0")))
    rng = np.random.default_rng(12)
    print(f"bench share: oracle dq on every tile of {cfg.heads} heads", flush=True)
    _dq_every_tile(host, dev, rng, [0, 1, L - 1])

    blocks = sorted(host.kv)
    k_pos = np.concatenate([oracle.positions(b, L) for b in blocks])
    for h in sorted(rng.choice(cfg.heads, size=4, replace=False).tolist()):
        local = sorted({0, 63, 64, 255, 256, L - 65, L - 64, L - 1} |
                       {t + int(rng.integers(128)) for t in range(0, L, 128)})
        keys = [b * L + j for b in blocks for j in local]
        k = torch.cat([host.kv[b][0][:, [h]] for b in blocks], dim=2)
        v = torch.cat([host.kv[b][1][:, [h]] for b in blocks], dim=2)
        print(f"bench share: oracle dk/dv of head {h} at {len(keys)} keys", flush=True)
        dk_ref, dv_ref = oracle.attention_grads_at_keys(
            host.q[:, [h]], k, v, host.dout[:, [h]], oracle.positions(rank, L), k_pos, True, keys)
        for i, b in enumerate(blocks):
            sel = slice(i * len(local), (i + 1) * len(local))
            got = dev.dkv_pool[b][:, :, [h]][:, :, :, local].cpu()
            check(f"dk[{b}] h{h}", got[0], dk_ref[:, :, sel], "bf16")
            check(f"dv[{b}] h{h}", got[1], dv_ref[:, :, sel], "bf16")
    assert torch.isfinite(dev.dq_acc).all()
