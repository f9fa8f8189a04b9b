"""The allocation-free decode step (ring_attn_fwd_decode_noalloc), through the
C ABI, against ring_attn_fwd_decode with caller-allocated split partials
and against the fp64 oracle.

Two calls in a row on one GPU, the second with a smaller input, so the
second call runs on a scratch array that still holds the first call's
partials: the results must not depend on them.  Same kernels and the same
key split on both paths, so the two entry points must agree bitwise; the
oracle gate is the one every decode test uses."""
import numpy as np
import pytest
import torch

import oracle
from blockwise_ring_attention_amd import _lib
from blockwise_ring_attention_amd.configs import DECODE_CONFIGS, DecodeConfig
from blockwise_ring_attention_amd.inputs import draw_decode
from tests._gates import check, check_lse

pytestmark = pytest.mark.gpu


def _oracle(cfg, q, kvs):
    Lk = cfg.kv_len
    k_pos = np.concatenate([oracle.positions(i, Lk) for i in range(len(kvs))])
    q_pos = oracle.positions(len(kvs), Lk, cfg.q_len)  # after every key
    B, H, Hkv = cfg.batch, cfg.heads, cfg.n_kv_heads
    G = H // Hkv
    o = np.zeros((B, H, cfg.q_len, cfg.head_dim))
    lse = np.zeros((B, H, cfg.q_len))
    for b in range(B):
        for kh in range(Hkv):
            k = torch.cat([kv[0, b:b + 1, kh:kh + 1] for kv in kvs], dim=2)
            v = torch.cat([kv[1, b:b + 1, kh:kh + 1] for kv in kvs], dim=2)
            ob, lb = oracle.attention(q[b:b + 1, kh * G:(kh + 1) * G], k, v, q_pos, k_pos,
                                      True, scale=cfg.scale or None)
            o[b, kh * G:(kh + 1) * G] = ob[0]
            lse[b, kh * G:(kh + 1) * G] = lb[0]
    return o, lse


def _both(cfg, q, kvs, k_chunk):
    """(o, lse) of the allocating and of the allocation-free entry point."""
    dev = torch.device("cuda:0")
    qd = q.to(dev)
    outs = []
    for noalloc in (False, True):
        o_acc = torch.empty(q.shape, dtype=torch.float32, device=dev)
        lse_acc = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        _lib.ring_attn_init_acc(o_acc, lse_acc)
        for kv in kvs:
            kvd = kv.to(dev)
            kc = k_chunk or _lib.ring_attn_decode_chunk(qd, kvd, cfg.scale)
            if noalloc:
                _lib.ring_attn_fwd_decode_noalloc(qd, kvd, kc, o_acc, lse_acc, cfg.scale)
            else:
                S = _lib.ring_attn_decode_splits(qd, kvd, kc, cfg.scale)
                o_part = torch.empty((S,) + tuple(q.shape), dtype=torch.float32, device=dev)
                lse_part = torch.empty((S,) + tuple(q.shape[:3]), dtype=torch.float32,
                                       device=dev)
                _lib.ring_attn_fwd_decode(qd, kvd, kc, o_acc, lse_acc, o_part, lse_part,
                                          cfg.scale)
        torch.cuda.synchronize()
        outs.append((o_acc.cpu(), lse_acc.cpu()))
    return outs


def test_noalloc_decode_matches_the_allocating_step_on_two_calls():
    big = DECODE_CONFIGS["decode-lwm7b"]        # 8 x 32 rows, 16384 keys, 2 splits
    small = DecodeConfig(97, "small after big", 2, 4, 128, 3, 1000, blocks=2, kv_heads=2,
                         k_chunk=200)           # ragged splits, grouped heads
    for cfg, seed in ((big, 0), (small, 3)):
        print(f"{cfg.name}: B {cfg.batch} H {cfg.heads} Lq {cfg.q_len} Lk {cfg.kv_len}",
              flush=True)
        q, kvs = draw_decode(cfg, seed=seed)
        (o_a, lse_a), (o_n, lse_n) = _both(cfg, q, kvs, cfg.k_chunk)
        assert torch.equal(o_n, o_a), f"{cfg.name}: o differs from ring_attn_fwd_decode"
        assert torch.equal(lse_n, lse_a), f"{cfg.name}: lse differs from ring_attn_fwd_decode"
        o_ref, lse_ref = _oracle(cfg, q, kvs)
        check(f"{cfg.name} o_acc", o_n, o_ref, "bf16")
        check_lse(f"{cfg.name} lse_acc", lse_n, lse_ref)


def test_noalloc_decode_rejects_more_splits_than_the_scratch_holds():
    dev = torch.device("cuda:0")
    # 8 x 32 rows, 200 splits of one key: 200 * 256 * 129 * 4 bytes > 16 MiB
    q = torch.zeros((8, 32, 1, 128), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((2, 8, 32, 200, 128), dtype=torch.bfloat16, device=dev)
    o_acc = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    lse_acc = torch.full(q.shape[:3], -float("inf"), dtype=torch.float32, device=dev)
    with pytest.raises(_lib.RingAttnError, match="scratch"):
        _lib.ring_attn_fwd_decode_noalloc(q, kv, 1, o_acc, lse_acc)
    torch.cuda.synchronize()
    assert torch.all(lse_acc == -float("inf")) and torch.all(o_acc == 0)
