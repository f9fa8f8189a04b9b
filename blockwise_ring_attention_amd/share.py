"""Run one ring member's whole share through the HIP library.

Host inputs come from ``inputs`` (seeded, one stream per global block); this
module uploads them, owns the device buffers of the single-GPU ring emulator
(member's queries, the pool of the other members' key/value blocks, two
receive slots, the fp32 accumulators) and calls the C ABI.  Every step of the
computation runs in the HIP kernels.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

from . import _lib
from .configs import ShareConfig
from .inputs import draw, draw_kv


@dataclass
class HostShare:
    """Host (CPU) tensors of one member's share."""
    cfg: ShareConfig
    rank: int
    q: torch.Tensor
    kv: Dict[int, torch.Tensor]          # global block id -> [2, B, H, L, d]
    dout: Optional[torch.Tensor] = None


def make_host_share(cfg: ShareConfig, rank: int, seed: int = 0, backward: bool = False,
                    workers: int = 8) -> HostShare:
    """Draw the member's queries and every key/value block it can see."""
    blocks = cfg.kv_blocks_seen(rank)
    with ThreadPoolExecutor(workers) as ex:
        fq = ex.submit(draw, cfg, "q", rank, seed)
        fd = ex.submit(draw, cfg, "do", rank, seed) if backward else None
        fkv = {b: ex.submit(draw_kv, cfg, b, seed) for b in blocks}
        kv = {b: f.result() for b, f in fkv.items()}
        return HostShare(cfg, rank, fq.result(), kv, fd.result() if fd else None)


@dataclass
class DeviceShare:
    cfg: ShareConfig
    rank: int
    q: torch.Tensor
    pool: List[Optional[torch.Tensor]]
    slots: List[torch.Tensor]
    o_acc: torch.Tensor
    lse_acc: torch.Tensor
    dout: Optional[torch.Tensor] = None
    delta: Optional[torch.Tensor] = None
    dq_acc: Optional[torch.Tensor] = None
    dkv_pool: List[Optional[torch.Tensor]] = field(default_factory=list)
    dkv_slots: List[torch.Tensor] = field(default_factory=list)
    work: Optional[torch.Tensor] = None  # dK/dV workspace for shared key/value heads


def upload(host: HostShare, device: str = "cuda") -> DeviceShare:
    cfg = host.cfg
    N = cfg.ring_size
    q = host.q.to(device)
    pool: List[Optional[torch.Tensor]] = [None] * N
    for b, t in host.kv.items():
        pool[b] = t.to(device)
    ref = next(t for t in pool if t is not None)
    slots = [torch.empty_like(ref), torch.empty_like(ref)]
    B, H, L, d = q.shape
    o_acc = torch.empty((B, H, L, d), dtype=torch.float32, device=device)
    lse_acc = torch.empty((B, H, L), dtype=torch.float32, device=device)
    dev = DeviceShare(cfg, host.rank, q, pool, slots, o_acc, lse_acc)
    if host.dout is not None:
        dev.dout = host.dout.to(device)
        dev.delta = torch.empty((B, H, L), dtype=torch.float32, device=device)
        dev.dq_acc = torch.empty((B, H, L, d), dtype=torch.float32, device=device)
        dev.dkv_pool = [None if t is None else torch.zeros(t.shape, dtype=torch.float32,
                                                           device=device) for t in pool]
        dev.dkv_slots = [torch.empty(ref.shape, dtype=torch.float32, device=device)
                         for _ in range(2)]
        nbytes = _lib.ring_attn_bwd_workspace(q, ref)
        if nbytes > 0:
            dev.work = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return dev


_side_streams: Dict[int, torch.cuda.Stream] = {}


def side_stream_for(device) -> torch.cuda.Stream:
    """One default-priority side stream per device for the emulated hops."""
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    if idx not in _side_streams:
        _side_streams[idx] = torch.cuda.Stream(device=idx)
    return _side_streams[idx]


def forward(dev: DeviceShare, q_chunk: Optional[int] = None, k_chunk: Optional[int] = None,
            order=None, serialize: bool = False, side_stream=None, unsafe: bool = False) -> None:
    """Initialise the accumulators and fold every block the member sees
    (unsafe: the emulator's race negative control, wrong results on purpose)."""
    cfg = dev.cfg
    if side_stream is None and not serialize:
        side_stream = side_stream_for(dev.q.device)
    _lib.ring_attn_init_acc(dev.o_acc, dev.lse_acc)
    _lib.ring_emu_fwd(dev.q, dev.pool, dev.slots, dev.rank, cfg.ring_size, cfg.causal,
                      q_chunk or cfg.q_chunk, k_chunk or cfg.k_chunk, dev.o_acc, dev.lse_acc,
                      order=order, serialize=serialize, side_stream=side_stream,
                      unsafe=unsafe)


def backward(dev: DeviceShare, q_chunk: Optional[int] = None, k_chunk: Optional[int] = None,
             order=None, serialize: bool = False, side_stream=None,
             use_work: bool = True, unsafe: bool = False) -> None:
    """Gradients of the finished forward share: dq_acc, and dkv_pool[kb] +=
    this member's dK/dV contribution for every block it sees.  With shared
    key/value heads the share's workspace (if any) lets query heads of a
    group run side by side (use_work=False: one after another)."""
    cfg = dev.cfg
    if side_stream is None and not serialize:
        side_stream = side_stream_for(dev.q.device)
    _lib.ring_attn_bwd_prep(dev.o_acc, dev.dout, dev.delta)
    dev.dq_acc.zero_()
    _lib.ring_emu_bwd(dev.q, dev.pool, dev.slots, dev.dout, dev.lse_acc, dev.delta,
                      dev.dkv_pool, dev.dkv_slots, dev.rank, cfg.ring_size, cfg.causal,
                      q_chunk or cfg.q_chunk, k_chunk or cfg.k_chunk, dev.dq_acc,
                      order=order, serialize=serialize, side_stream=side_stream,
                      work=dev.work if use_work else None, unsafe=unsafe)


def finalize(dev: DeviceShare) -> torch.Tensor:
    """The member's output in the input dtype (bf16 with RNE, or fp32)."""
    out = torch.empty(dev.o_acc.shape, dtype=dev.q.dtype, device=dev.q.device)
    _lib.ring_attn_finalize(dev.o_acc, out)
    return out
