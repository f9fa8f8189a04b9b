"""GPU parity of the decode-shaped step (ring_attn_fwd_decode) against the
fp64 oracle, through the C ABI.

The query rows come after every key, so the oracle is exact causal attention
with the queries placed after the last key block (which masks nothing), over
all the key/value blocks the step folds in, one after another.  Small cases
are compared element by element; they span several key tiles, ragged splits,
one and two blocks of 32 rows per key/value head group, d = 64 and 128, and
the degenerate splits (one key per split, a single split).  The full-size
decode workload, with the key split the benchmark uses, is compared on every
row."""
import numpy as np
import pytest
import torch

import oracle
from blockwise_ring_attention_amd import _lib
from blockwise_ring_attention_amd.configs import DECODE_CONFIGS, DecodeConfig, Dist
from blockwise_ring_attention_amd.inputs import draw_decode
from tests._gates import check, check_lse

pytestmark = pytest.mark.gpu


def _oracle(cfg, q, kvs, heads=None):
    """Oracle o, lse [B, H, Lq(, d)], one key/value head at a time so that only
    that head's keys are upcast to float64."""
    Lk = cfg.kv_len
    k_pos = np.concatenate([oracle.positions(i, Lk) for i in range(len(kvs))])
    q_pos = oracle.positions(len(kvs), Lk, cfg.q_len)   # after every key
    B, H = cfg.batch, cfg.heads
    Hkv = cfg.n_kv_heads
    G = H // Hkv
    o = np.zeros((B, H, cfg.q_len, cfg.head_dim))
    lse = np.zeros((B, H, cfg.q_len))
    for b in range(B):
        for kh in range(Hkv):
            k = torch.cat([kv[0, b:b + 1, kh:kh + 1] for kv in kvs], dim=2)
            v = torch.cat([kv[1, b:b + 1, kh:kh + 1] for kv in kvs], dim=2)
            qh = q[b:b + 1, kh * G:(kh + 1) * G]
            ob, lb = oracle.attention(qh, k, v, q_pos, k_pos, True,
                                      scale=cfg.scale or None)
            o[b, kh * G:(kh + 1) * G] = ob[0]
            lse[b, kh * G:(kh + 1) * G] = lb[0]
    return o, lse


def _run(cfg, q, kvs, k_chunk=None):
    dev = torch.device("cuda:0")
    qd = q.to(dev)
    o_acc = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse_acc = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    _lib.ring_attn_init_acc(o_acc, lse_acc)
    for kv in kvs:
        kvd = kv.to(dev)
        kc = k_chunk or cfg.k_chunk or _lib.ring_attn_decode_chunk(qd, kvd, cfg.scale)
        S = _lib.ring_attn_decode_splits(qd, kvd, kc, cfg.scale)
        o_part = torch.empty((max(S, 1),) + tuple(q.shape), dtype=torch.float32, device=dev)
        lse_part = torch.empty((max(S, 1),) + tuple(q.shape[:3]), dtype=torch.float32,
                               device=dev)
        _lib.ring_attn_fwd_decode(qd, kvd, kc, o_acc, lse_acc, o_part, lse_part, cfg.scale)
    torch.cuda.synchronize()
    return o_acc.cpu(), lse_acc.cpu()


SMALL = [
    # (name, B, H, Hkv, d, Lq, Lk, blocks, k_chunk, scale)
    ("mha one row, ragged splits, two blocks", 2, 4, 0, 128, 1, 1000, 2, 200, 0.0),
    ("gqa 8 heads x 4 rows = 32 per group", 1, 16, 2, 128, 4, 777, 1, 256, 0.05),
    ("mqa 8 heads x 8 rows = 64 per group", 2, 8, 1, 128, 8, 1500, 2, 0, 0.0),
    ("d64 mqa 40 rows per group", 1, 8, 1, 64, 5, 333, 1, 100, 0.0),
    ("d64 mha one row", 2, 3, 0, 64, 1, 640, 2, 0, 0.0),
    ("33 rows, one head per group", 1, 2, 0, 128, 33, 300, 1, 128, 0.0),
    ("one key per split", 1, 2, 0, 128, 3, 70, 1, 1, 0.0),
    ("single split over the whole block", 1, 2, 2, 128, 2, 129, 1, 4096, 0.0),
    ("ten blocks of 64 keys", 1, 4, 2, 128, 2, 64, 10, 64, 0.0),
    ("a single key, three blocks", 2, 4, 1, 64, 3, 1, 3, 0, 0.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_decode_small_elementwise(case):
    name, B, H, Hkv, d, Lq, Lk, blocks, kc, scale = case
    print(name, flush=True)
    cfg = DecodeConfig(92, name, B, H, d, Lq, Lk, blocks=blocks, kv_heads=Hkv, k_chunk=kc,
                       scale=scale)
    q, kvs = draw_decode(cfg, seed=5)
    o, lse = _run(cfg, q, kvs)
    o_ref, lse_ref = _oracle(cfg, q, kvs)
    check("o_acc", o, o_ref, "bf16")
    check_lse("lse_acc", lse, lse_ref)


def test_decode_adversarial_scores():
    """Scores with standard deviation ~100 stress the running-max rescale
    inside a split and the fold across splits."""
    cfg = DecodeConfig(93, "adv", 1, 4, 128, 2, 2048, blocks=2, kv_heads=2, k_chunk=512,
                       dists={"q": Dist("normal", 3.0), "k": Dist("normal", 3.0),
                              "v": Dist("uniform", 1.0)})
    q, kvs = draw_decode(cfg, seed=1)
    o, lse = _run(cfg, q, kvs)
    o_ref, lse_ref = _oracle(cfg, q, kvs)
    check("o_acc", o, o_ref, "bf16")
    check_lse("lse_acc", lse, lse_ref)


def test_decode_split_invariance():
    """The key split changes only rounding: three splits against the oracle."""
    cfg = DecodeConfig(94, "splits", 1, 4, 128, 1, 4096, kv_heads=1)
    q, kvs = draw_decode(cfg, seed=2)
    o_ref, lse_ref = _oracle(cfg, q, kvs)
    for kc in (64, 1000, 4096):
        print(f"k_chunk {kc}", flush=True)
        o, lse = _run(cfg, q, kvs, k_chunk=kc)
        check(f"o_acc k_chunk={kc}", o, o_ref, "bf16")
        check_lse(f"lse_acc k_chunk={kc}", lse, lse_ref)


def test_decode_empty_block_leaves_accumulators_unchanged():
    dev = torch.device("cuda:0")
    cfg = DecodeConfig(95, "empty", 1, 2, 128, 1, 256)
    q, kvs = draw_decode(cfg, seed=0)
    o0, lse0 = _run(cfg, q, kvs)
    qd = q.to(dev)
    o_acc, lse_acc = o0.to(dev), lse0.to(dev)
    empty = torch.empty((2, 1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    part = torch.empty((1,) + tuple(q.shape), dtype=torch.float32, device=dev)
    lpart = torch.empty((1,) + tuple(q.shape[:3]), dtype=torch.float32, device=dev)
    _lib.ring_attn_fwd_decode(qd, empty, 64, o_acc, lse_acc, part, lpart)
    torch.cuda.synchronize()
    assert torch.equal(o_acc.cpu(), o0) and torch.equal(lse_acc.cpu(), lse0)


@pytest.mark.parametrize("kv_heads", [0, 8], ids=["mha", "gqa4"])
def test_decode_full_size_every_row(kv_heads):
    """The decode workload the benchmark times (8 sequences, 32 heads of 128,
    16384 keys), with the library's own key split, on every row."""
    base = DECODE_CONFIGS["decode-lwm7b"]
    from dataclasses import replace
    cfg = replace(base, kv_heads=kv_heads)
    print(f"{cfg.name} kv_heads {cfg.n_kv_heads}", flush=True)
    q, kvs = draw_decode(cfg, seed=0)
    o, lse = _run(cfg, q, kvs)
    o_ref, lse_ref = _oracle(cfg, q, kvs)
    check("o_acc", o, o_ref, "bf16")
    check_lse("lse_acc", lse, lse_ref)


def test_speculative_step_composes_with_the_causal_diagonal_step():
    """A short run of draft rows: they attend to every cached key through the
    decode step, then to their own new keys through the ordinary causal
    diagonal ring step; together that is exact causal attention over the
    cache and the draft (grouped key/value heads, d = 128)."""
    from blockwise_ring_attention_amd.inputs import draw
    dev = torch.device("cuda:0")
    cfg = DecodeConfig(96, "draft", 2, 8, 128, 8, 1000, blocks=2, kv_heads=2)
    q, kvs = draw_decode(cfg, seed=7)
    kv_draft = torch.stack([draw(cfg, "k", cfg.blocks, 7, length=cfg.q_len),
                            draw(cfg, "v", cfg.blocks, 7, length=cfg.q_len)], dim=0)
    qd = q.to(dev)
    o_acc = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse_acc = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    _lib.ring_attn_init_acc(o_acc, lse_acc)
    for kv in kvs:
        kvd = kv.to(dev)
        kc = _lib.ring_attn_decode_chunk(qd, kvd)
        S = _lib.ring_attn_decode_splits(qd, kvd, kc)
        o_part = torch.empty((S,) + tuple(q.shape), dtype=torch.float32, device=dev)
        lse_part = torch.empty((S,) + tuple(q.shape[:3]), dtype=torch.float32, device=dev)
        _lib.ring_attn_fwd_decode(qd, kvd, kc, o_acc, lse_acc, o_part, lse_part)
    # the draft block is the member's own block: ring step 0, causal diagonal
    _lib.ring_attn_fwd(qd, kv_draft.to(dev), 2, 0, 3, True, 256, 64, o_acc, lse_acc)
    torch.cuda.synchronize()

    Lk, G = cfg.kv_len, cfg.heads // cfg.n_kv_heads
    k_pos = np.concatenate([oracle.positions(0, Lk), oracle.positions(1, Lk),
                            2 * Lk + np.arange(cfg.q_len)])
    q_pos = 2 * Lk + np.arange(cfg.q_len)
    o_ref = np.zeros(q.shape)
    lse_ref = np.zeros(q.shape[:3])
    for b in range(cfg.batch):
        for kh in range(cfg.n_kv_heads):
            k = torch.cat([kvs[0][0, b:b + 1, kh:kh + 1], kvs[1][0, b:b + 1, kh:kh + 1],
                           kv_draft[0, b:b + 1, kh:kh + 1]], dim=2)
            v = torch.cat([kvs[0][1, b:b + 1, kh:kh + 1], kvs[1][1, b:b + 1, kh:kh + 1],
                           kv_draft[1, b:b + 1, kh:kh + 1]], dim=2)
            ob, lb = oracle.attention(q[b:b + 1, kh * G:(kh + 1) * G], k, v, q_pos, k_pos, True)
            o_ref[b, kh * G:(kh + 1) * G] = ob[0]
            lse_ref[b, kh * G:(kh + 1) * G] = lb[0]
    check("o_acc", o_acc.cpu(), o_ref, "bf16")
    check_lse("lse_acc", lse_acc.cpu(), lse_ref)
