"""The entry points can be captured into a HIP graph (they enqueue only on
the caller's stream, allocate nothing and clear with fill kernels, not
memsets): each captured sequence is replayed several times, with the
program's own eager work and synchronisations in between, and every replay
must equal the eager result bitwise."""
import pytest
import torch

from blockwise_ring_attention_amd import _lib, share
from blockwise_ring_attention_amd.configs import DecodeConfig, FfnConfig, ShareConfig
from blockwise_ring_attention_amd.inputs import draw_decode, draw_ffn, draw_ffn_dout

pytestmark = pytest.mark.gpu


def _capture_and_replay(step, outputs, scribble, replays=3):
    """Run step eagerly, capture it, then replay it `replays` times after
    scribbling over the outputs; return True if every replay matches."""
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                      # warm-up on the capture stream's kind
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(replays):
        scribble(i)                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(o, r), f"replay {i} differs from the eager result"


def test_decode_step_in_a_graph():
    dev = torch.device("cuda:0")
    cfg = DecodeConfig(97, "graph", 2, 8, 128, 2, 700, blocks=2, kv_heads=2)
    q, kvs = draw_decode(cfg, seed=3)
    qd = q.to(dev)
    kvd = [kv.to(dev) for kv in kvs]
    o_acc = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse_acc = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    kc = _lib.ring_attn_decode_chunk(qd, kvd[0])
    S = _lib.ring_attn_decode_splits(qd, kvd[0], kc)
    o_part = torch.empty((S,) + tuple(q.shape), dtype=torch.float32, device=dev)
    lse_part = torch.empty((S,) + tuple(q.shape[:3]), dtype=torch.float32, device=dev)

    def step():
        _lib.ring_attn_init_acc(o_acc, lse_acc)
        for kv in kvd:
            _lib.ring_attn_fwd_decode(qd, kv, kc, o_acc, lse_acc, o_part, lse_part)

    def scribble(i):
        o_acc.fill_(float(i + 1))
        lse_acc.fill_(-float(i + 1))
        o_part.fill_(7.0)

    _capture_and_replay(step, [o_acc, lse_acc], scribble)


def test_causal_forward_share_in_a_graph():
    dev = torch.device("cuda:0")
    cfg = ShareConfig(98, "graph", "bf16", 1, 2, 128, 3, 320, (2,), True, 256, 64)
    host = share.make_host_share(cfg, 2, seed=4)
    q = host.q.to(dev)
    blocks = {b: host.kv[b].to(dev) for b in host.kv}
    o_acc = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse_acc = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)

    def step():
        _lib.ring_attn_init_acc(o_acc, lse_acc)
        for s in range(cfg.ring_size):
            kb = (2 - s) % cfg.ring_size
            _lib.ring_attn_fwd(q, blocks[kb], 2, s, cfg.ring_size, True, cfg.q_chunk,
                               cfg.k_chunk, o_acc, lse_acc)
        _lib.ring_attn_finalize(o_acc, out)

    def scribble(i):
        o_acc.fill_(3.0)
        out.fill_(-1.0)

    _capture_and_replay(step, [o_acc, lse_acc, out], scribble)


def test_feedforward_in_a_graph():
    dev = torch.device("cuda:0")
    cfg = FfnConfig(99, "graph", rows=300, d_model=256, d_ff=512, chunk_rows=128)
    x, w1, w2 = (t.to(dev) for t in draw_ffn(cfg, seed=5))
    hidden = torch.empty((128, 512), dtype=torch.bfloat16, device=dev)
    out = torch.empty((300, 256), dtype=torch.bfloat16, device=dev)

    def step():
        _lib.ring_ffn_fwd(x, w1, w2, hidden, out, cfg.chunk_rows)

    def scribble(i):
        out.fill_(float(i))

    _capture_and_replay(step, [out], scribble)


def test_causal_backward_share_in_a_graph():
    """Delta preparation and the three ring steps of the backward (dQ and the
    travelling dK/dV partials cleared by fill kernels inside the graph)."""
    dev = torch.device("cuda:0")
    cfg = ShareConfig(98, "graph", "bf16", 1, 4, 128, 3, 320, (2,), True, 256, 64,
                      backward=True, kv_heads=2)
    host = share.make_host_share(cfg, 2, seed=6, backward=True)
    q, dout = host.q.to(dev), host.dout.to(dev)
    blocks = {b: host.kv[b].to(dev) for b in host.kv}
    o_acc = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse_acc = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    _lib.ring_attn_init_acc(o_acc, lse_acc)
    for s in range(cfg.ring_size):
        _lib.ring_attn_fwd(q, blocks[(2 - s) % 3], 2, s, 3, True, cfg.q_chunk, cfg.k_chunk,
                           o_acc, lse_acc)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dkv = {b: torch.empty(t.shape, dtype=torch.float32, device=dev) for b, t in blocks.items()}

    def step():
        dq.zero_()
        for t in dkv.values():
            t.zero_()
        _lib.ring_attn_bwd_prep(o_acc, dout, delta)
        for s in range(cfg.ring_size):
            kb = (2 - s) % 3
            _lib.ring_attn_bwd(q, blocks[kb], dout, lse_acc, delta, 2, s, 3, True,
                               cfg.q_chunk, cfg.k_chunk, dq, dkv[kb])

    def scribble(i):
        dq.fill_(5.0)
        delta.fill_(-2.0)
        for t in dkv.values():
            t.fill_(float(i))

    _capture_and_replay(step, [delta, dq] + list(dkv.values()), scribble)


def test_feedforward_backward_in_a_graph():
    dev = torch.device("cuda:0")
    cfg = FfnConfig(99, "graph", rows=300, d_model=256, d_ff=512, chunk_rows=128)
    x, w1, w2 = (t.to(dev) for t in draw_ffn(cfg, seed=7))
    dout = draw_ffn_dout(cfg, seed=7).to(dev)
    dx = torch.empty((300, 256), dtype=torch.bfloat16, device=dev)
    dw1 = torch.empty((512, 256), dtype=torch.float32, device=dev)
    dw2 = torch.empty((256, 512), dtype=torch.float32, device=dev)
    work = torch.empty(_lib.ring_ffn_bwd_workspace(300, 256, 512, cfg.chunk_rows),
                       dtype=torch.uint8, device=dev)

    def step():
        dw1.zero_()
        dw2.zero_()
        _lib.ring_ffn_bwd(x, w1, w2, dout, dx, dw1, dw2, work, cfg.chunk_rows)

    def scribble(i):
        dx.fill_(float(i))
        dw1.fill_(1.0)
        work.fill_(0x7f)

    _capture_and_replay(step, [dx, dw1, dw2], scribble)
