"""GPU parity of the forward ring share against the fp64 oracle, through the
C ABI.  Small cases are compared element by element (several tiles and a
ragged tail); the full-size workloads, in the launch configuration the
benchmark times, are compared on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from blockwise_ring_attention_amd import _lib, share
from blockwise_ring_attention_amd.configs import CONFIGS, ShareConfig, Dist, scaled
from tests._gates import check, check_lse, oracle_rows, oracle_rows_per_head, seam_rows, tile_rows

pytestmark = pytest.mark.gpu


def _full_oracle(host):
    cfg = host.cfg
    L = cfg.block_len
    blocks = sorted(host.kv)
    k = torch.cat([host.kv[b][0] for b in blocks], dim=2)
    v = torch.cat([host.kv[b][1] for b in blocks], dim=2)
    k_pos = np.concatenate([oracle.positions(b, L) for b in blocks])
    return oracle.attention(host.q, k, v, oracle.positions(host.rank, L), k_pos, cfg.causal)


def _run(host, **kw):
    dev = share.upload(host)
    share.forward(dev, **kw)
    out = share.finalize(dev)
    torch.cuda.synchronize()
    return dev, out


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_cfg1_tiny_exact_fp32_all_ranks(rank):
    cfg = CONFIGS[1]
    print(f"cfg1 rank {rank}", flush=True)
    host = share.make_host_share(cfg, rank)
    dev, out = _run(host)
    o_ref, lse_ref = _full_oracle(host)
    check("o_acc", dev.o_acc, o_ref, "fp32")
    check("o", out, o_ref, "fp32")
    check_lse("lse", dev.lse_acc, lse_ref)


SMALL = [
    # (name, dtype, B, H, d, N, L, rank, causal, q_chunk, k_chunk)
    ("bf16 d128 causal ragged", "bf16", 1, 2, 128, 3, 300, 2, True, 256, 64),
    ("bf16 d128 causal narrow tiles", "bf16", 2, 1, 128, 2, 200, 1, True, 128, 32),
    ("bf16 d64 causal", "bf16", 1, 3, 64, 4, 160, 3, True, 256, 64),
    ("bf16 d64 noncausal", "bf16", 1, 2, 64, 3, 96, 0, False, 128, 32),
    ("bf16 d128 noncausal rank1", "bf16", 2, 2, 128, 4, 130, 1, False, 256, 64),
    ("bf16 d128 diagonal only, three workgroups", "bf16", 1, 2, 128, 2, 600, 0, True, 256, 64),
    ("fp32 d128 causal ragged", "fp32", 1, 2, 128, 3, 100, 2, True, 64, 64),
    ("fp32 d64 noncausal", "fp32", 1, 2, 64, 2, 77, 1, False, 64, 64),
    # degenerate lengths: one token per block, and one row past a 32-row tile
    ("bf16 d128 causal single token", "bf16", 1, 2, 128, 3, 1, 2, True, 256, 64),
    ("bf16 d64 noncausal 33 tokens", "bf16", 1, 2, 64, 2, 33, 1, False, 128, 32),
    ("fp32 d128 causal single token", "fp32", 1, 1, 128, 2, 1, 1, True, 64, 64),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shares_elementwise(case):
    name, dtype, B, H, d, N, L, rank, causal, qc, kc = case
    print(name, flush=True)
    cfg = ShareConfig(90, name, dtype, B, H, d, N, L, (rank,), causal, qc, kc)
    host = share.make_host_share(cfg, rank, seed=3)
    dev, out = _run(host)
    o_ref, lse_ref = _full_oracle(host)
    check("o_acc", dev.o_acc, o_ref, dtype)
    check_lse("lse", dev.lse_acc, lse_ref)


def test_adversarial_scores_small():
    """Scores with standard deviation ~100 stress the running-max rescale."""
    cfg = ShareConfig(91, "adv", "bf16", 1, 2, 128, 4, 192, (3,), True, 256, 64,
                      dists={"q": Dist("normal", 3.0), "k": Dist("normal", 3.0),
                             "v": Dist("uniform", 1.0)})
    host = share.make_host_share(cfg, 3)
    dev, _ = _run(host)
    o_ref, lse_ref = _full_oracle(host)
    check("o_acc", dev.o_acc, o_ref, "bf16")
    check_lse("lse", dev.lse_acc, lse_ref)


def test_chunk_sizes_do_not_change_the_result():
    cfg = ShareConfig(92, "chunks", "bf16", 1, 2, 128, 2, 256, (1,), True, 256, 64)
    host = share.make_host_share(cfg, 1)
    o_ref, lse_ref = _full_oracle(host)
    for qc, kc in ((256, 64), (128, 64), (256, 32), (64, 32), (1024, 1024)):
        dev, _ = _run(host, q_chunk=qc, k_chunk=kc)
        check(f"o qc={qc} kc={kc}", dev.o_acc, o_ref, "bf16")
        check_lse(f"lse qc={qc} kc={kc}", dev.lse_acc, lse_ref)


def test_per_step_calls_match_emulator_bitwise_and_future_is_noop():
    cfg = ShareConfig(93, "steps", "bf16", 1, 2, 128, 4, 128, (2,), True, 256, 64)
    host = share.make_host_share(cfg, 2)
    dev, _ = _run(host)
    q = host.q.cuda()
    o = torch.empty_like(dev.o_acc)
    lse = torch.empty_like(dev.lse_acc)
    _lib.ring_attn_init_acc(o, lse)
    for s in range(cfg.ring_size):
        kb = (2 - s) % cfg.ring_size
        kv = host.kv[kb].cuda() if kb in host.kv else torch.full_like(host.kv[0].cuda(), float("nan"))
        before = (o.clone(), lse.clone())
        _lib.ring_attn_fwd(q, kv, 2, s, cfg.ring_size, True, 256, 64, o, lse)
        if kb > 2:   # future block: no launch, accumulators bitwise unchanged
            torch.cuda.synchronize()
            assert torch.equal(o, before[0]) and torch.equal(lse, before[1])
    torch.cuda.synchronize()
    assert torch.equal(o, dev.o_acc) and torch.equal(lse, dev.lse_acc)


def test_empty_block_and_empty_queries():
    q = torch.randn(1, 2, 64, 128, device="cuda").to(torch.bfloat16)
    kv0 = torch.empty(2, 1, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    o = torch.zeros(1, 2, 64, 128, device="cuda")
    lse = torch.full((1, 2, 64), float("-inf"), device="cuda")
    _lib.ring_attn_fwd(q, kv0, 0, 0, 1, False, 64, 64, o, lse)     # no keys: identity
    q0 = torch.empty(1, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    kv = torch.randn(2, 1, 2, 64, 128, device="cuda").to(torch.bfloat16)
    _lib.ring_attn_fwd(q0, kv, 0, 0, 1, False, 64, 64, torch.empty(1, 2, 0, 128, device="cuda"),
                       torch.empty(1, 2, 0, device="cuda"))
    torch.cuda.synchronize()
    assert (o == 0).all() and torch.isneginf(lse).all()


def test_invalid_arguments_raise_without_launch():
    q = torch.randn(1, 1, 64, 128, device="cuda").to(torch.bfloat16)
    kv = torch.randn(2, 1, 1, 64, 128, device="cuda").to(torch.bfloat16)
    o = torch.zeros(1, 1, 64, 128, device="cuda")
    lse = torch.full((1, 1, 64), float("-inf"), device="cuda")
    with pytest.raises(_lib.RingAttnError, match="ring_rank"):
        _lib.ring_attn_fwd(q, kv, 3, 0, 2, True, 64, 64, o, lse)
    kv_short = torch.randn(2, 1, 1, 32, 128, device="cuda").to(torch.bfloat16)
    with pytest.raises(_lib.RingAttnError, match="equal blocks"):
        _lib.ring_attn_fwd(q, kv_short, 0, 0, 1, True, 64, 64, o, lse)
    torch.cuda.synchronize()
    assert (o == 0).all()


def test_combine_kernel_algebra():
    g = torch.Generator().manual_seed(0)
    shape = (2, 3, 50, 128)
    parts = []
    for _ in range(3):
        o = torch.randn(shape, generator=g)
        lse = torch.randn(shape[:-1], generator=g) * 4
        lse[..., :3] = float("-inf")
        o[..., :3, :] = 0
        parts.append((o, lse))
    a, b, c = parts
    ref = oracle.combine(*oracle.combine(*a, *b), *c)
    oa, la = a[0].cuda(), a[1].cuda()
    ob, lb = b[0].cuda(), b[1].cuda()
    oc, lc = c[0].cuda(), c[1].cuda()
    _lib.ring_attn_combine(oa, la, ob, lb)
    _lib.ring_attn_combine(oa, la, oc, lc)
    # the other association
    ob2, lb2 = b[0].cuda(), b[1].cuda()
    _lib.ring_attn_combine(ob2, lb2, oc, lc)
    oa2, la2 = a[0].cuda(), a[1].cuda()
    _lib.ring_attn_combine(oa2, la2, ob2, lb2)
    torch.cuda.synchronize()
    for o, l in ((oa, la), (oa2, la2)):
        np.testing.assert_allclose(o.cpu().numpy(), ref[0], atol=1e-5, rtol=1e-5)
        np.testing.assert_array_equal(np.isneginf(l.cpu().numpy()), np.isneginf(ref[1]))
        fin = np.isfinite(ref[1])
        np.testing.assert_allclose(l.cpu().numpy()[fin], ref[1][fin], atol=1e-5)


def _tile_parity(host, dev, out, tile, rng, seams):
    """Compare one row of every query tile of every head (plus seam rows) with
    the oracle: every workgroup the launch ran has a row checked."""
    cfg = host.cfg
    rows_of = {h: tile_rows(cfg.block_len, tile, rng, seams) for h in range(cfg.heads)}
    ref = oracle_rows_per_head(host, rows_of)
    for name, got_all in (("o_acc", dev.o_acc), ("o (bf16)", out)):
        got = torch.cat([got_all[:, h][:, rows_of[h]] for h in range(cfg.heads)], dim=1)
        want = np.concatenate([ref[h][0] for h in range(cfg.heads)], axis=1)
        check(name, got, want, "bf16")
    got = torch.cat([dev.lse_acc[:, h][:, rows_of[h]] for h in range(cfg.heads)], dim=1)
    check_lse("lse", got, np.concatenate([ref[h][1] for h in range(cfg.heads)], axis=1))
    return sum(len(r) for r in rows_of.values())


@pytest.mark.parametrize("cfg_id", [2, 3, 5])
def test_full_size_every_tile(cfg_id):
    """Full-size workloads at the benchmark's launch configuration (256-row
    query tiles), compared with the oracle on one random row of every tile of
    every head, plus block and chunk seam rows."""
    cfg = CONFIGS[cfg_id]
    rank = cfg.ranks[0]
    print(f"cfg{cfg_id} rank {rank}: generating inputs", flush=True)
    host = share.make_host_share(cfg, rank)
    print(f"cfg{cfg_id}: running share", flush=True)
    dev, out = _run(host)
    rng = np.random.default_rng(cfg_id)
    seams = seam_rows(cfg.block_len, cfg.q_chunk, rng, 0)
    n = _tile_parity(host, dev, out, 256, rng, seams)
    print(f"cfg{cfg_id}: {n} rows checked over {cfg.heads} heads x batch {cfg.batch}", flush=True)
    assert torch.isfinite(dev.o_acc).all() and torch.isfinite(dev.lse_acc).all()


@pytest.mark.parametrize("fault", ["dropped", "duplicated", "wrong block"])
def test_full_size_ring_faults_fail_the_gates(fault):
    """Negative controls at the 16384-query causal share (rank 7 of 8): a ring
    step that loses a past block, folds one twice, or receives block kb + 1 in
    place of kb must fail the parity gates (on o the 2e-2 absolute term alone
    would not notice: o has a standard deviation of about 1.3e-3 here; the
    relative Frobenius guard and the LSE gate do).  The untouched schedule
    passes the same gates on the same rows.  A wrong cross-chunk combine can
    leave attention quietly incorrect (darcstar commentary), so the gates
    must see it."""
    cfg = CONFIGS[3]
    rank, N = cfg.ranks[0], cfg.ring_size
    print(f"faults ({fault}): generating inputs", flush=True)
    host = share.make_host_share(cfg, rank)
    q = host.q.cuda()
    kvd = {b: t.cuda() for b, t in host.kv.items()}
    victim = 3                       # a past block
    rng = np.random.default_rng(31)
    heads = [0, 17]
    rows_of = {h: tile_rows(cfg.block_len, 512, rng) for h in heads}
    ref = oracle_rows_per_head(host, rows_of)

    def run(faulty):
        o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        _lib.ring_attn_init_acc(o, lse)
        for s in range(N):
            kb = (rank - s) % N
            blocks = [kb]
            if faulty and kb == victim:
                blocks = {"dropped": [], "duplicated": [kb, kb], "wrong block": [kb + 1]}[fault]
            for b in blocks:
                _lib.ring_attn_fwd(q, kvd[b], rank, s, N, True, cfg.q_chunk, cfg.k_chunk, o, lse)
        torch.cuda.synchronize()
        return o, lse

    def gates(o, lse):
        for h in heads:
            check(f"o h{h}", o[:, h][:, rows_of[h]], ref[h][0], "bf16")
            check_lse(f"lse h{h}", lse[:, h][:, rows_of[h]], ref[h][1])

    gates(*run(False))
    print(f"faults ({fault}): faulty schedule", flush=True)
    with pytest.raises(AssertionError, match="rel Frobenius|LSE"):
        gates(*run(True))


@pytest.mark.parametrize("kv_heads,dtype", [(1, "bf16"), (2, "bf16"), (2, "fp32")])
def test_shared_kv_heads_forward(kv_heads, dtype):
    """MQA / GQA: four query heads over one or two key/value heads, causal
    ragged share, element by element against the oracle."""
    cfg = ShareConfig(97, f"shared-kv{kv_heads}", dtype, 1, 4, 128, 3, 200, (2,), True,
                      256 if dtype == "bf16" else 64, 64, kv_heads=kv_heads)
    host = share.make_host_share(cfg, 2, seed=4)
    assert host.kv[0].shape[2] == kv_heads
    dev, _ = _run(host)
    o_ref, lse_ref = _full_oracle(host)
    check("o_acc", dev.o_acc, o_ref, dtype)
    check_lse("lse", dev.lse_acc, lse_ref)
