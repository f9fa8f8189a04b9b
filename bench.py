#!/usr/bin/env python3
"""Throughput of one ring member's attention share on one MI355X.

Workload: the LWM-7B-shaped causal share (batch 1, 32 heads, head_dim 128,
bf16, ring of 8, the last member: 16384 local queries against 131072 keys).
One step is the whole hot path: initialise the accumulators, fold the 8
key/value blocks in ring order through the single-GPU ring emulator (each
hop a device-to-device copy on a side stream, overlapped with compute),
cast the output to bf16, then the backward share (row dot products, then the
8 blocks again, each block's dK/dV partial received, accumulated and sent
on).  Inputs are resident in HBM before the timed region starts.

Throughput is causal-adjusted: 4*d flops per unmasked (query, key) pair for
the forward and 10*d for the backward (which recomputes the scores), over
r*L^2 + L(L+1)/2 pairs per head for member r with blocks of L tokens.

``--decode`` times the decode-shaped step instead: 8 sequences, one new
query row each, 32 heads of 128 (``--kv-heads`` for shared key/value heads),
against one member's 16384-token share of the key/value cache.  That step
streams the key/value block from HBM once, so it reports HBM GB/s of its
algorithmic bytes against the 8 TB/s peak.

``--ffn`` times a training step of the blockwise feedforward of one member's
16384-token block of the 7B model instead (width 4096, hidden 16384, 4096
rows per chunk): forward 4·rows·d_model·d_ff flops (two bf16 MFMA products
per chunk) and backward 10·rows·d_model·d_ff (the up-projection recomputed,
then dH, dx, dW1, dW2), weight gradients accumulating over the steps.

Prints one JSON line.  ``--gpus`` above 1 is refused: this benchmark runs one
member's share on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "causal-adjusted attention TFLOP/s per GPU (fwd, fwd+bwd); % of bf16 MFMA peak"
FWD_FLOPS_PER_PAIR_PER_D = 4
BWD_FLOPS_PER_PAIR_PER_D = 10
# Products each kernel family forms per unmasked pair, in units of d flops:
# forward S and PV; the backward's query-major dQ kernel forms S, dP and dQ,
# its key-major dK/dV kernel forms S, dP, dV and dK.
KERNEL_FLOPS_PER_PAIR_PER_D = {"fwd_bf16": 4, "bwd_dq": 6, "bwd_dkv": 8}


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the oracle's timed CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phases", action="store_true",
                    help="skip the separate forward-only / backward-only timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (a known amount of "
                         "HBM traffic, to scale the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--config", type=int, default=3,
                    help="attention workload: 3 (default) the 16384-query causal share with "
                         "its backward; 2 the non-causal share (forward); 4 the 8192-token "
                         "training share (forward + backward); 5 the million-token share "
                         "(forward)")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="key/value heads shared by groups of the 32 query heads (MQA / GQA); "
                         "0 (default): 32, ordinary multi-head attention")
    ap.add_argument("--decode", action="store_true",
                    help="time the decode-shaped step (few query rows against a long "
                         "key/value block; HBM-bound) instead of the training share")
    ap.add_argument("--ffn", action="store_true",
                    help="time the blockwise feedforward of the member's block instead")
    ap.add_argument("--trace-overlap", metavar="KERNEL_TRACE_CSV",
                    help="no GPU: read a rocprofv3 --kernel-trace CSV of this benchmark and "
                         "report how much of the ring-hop copy time overlaps the attention "
                         "kernels, then exit")
    return ap.parse_args()


# Kernel-name fragments of the attention kernels and of the emulated ring
# hop (hipMemcpyAsync device-to-device copies run as copy kernels).
_ATTN_KERNELS = ("fwd_bf16_kernel", "fwd_fp32_kernel", "dq_kernel", "dkv_kernel",
                 "decode_kernel", "fold_kernel", "gemm_tn_kernel")
_COPY_KERNEL = "copyBuffer"


def _trace_overlap(path):
    """Fraction of copy-kernel time during which an attention kernel runs."""
    import csv
    rows = list(csv.DictReader(open(path)))
    span = lambda r: (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    attn = sorted(span(r) for r in rows if any(k in r["Kernel_Name"] for k in _ATTN_KERNELS))
    copies = [r for r in rows if _COPY_KERNEL in r["Kernel_Name"]]
    total = covered = 0
    for r in copies:
        a, b = span(r)
        total += b - a
        # attention kernels run one at a time on the main stream: no double count
        covered += sum(min(b, e) - max(a, s) for s, e in attn if s < b and e > a)
    print(json.dumps({
        "copy_kernels": len(copies),
        "copy_ms": round(total / 1e6, 3),
        "copy_ms_overlapped_by_attention": round(covered / 1e6, 3),
        "overlap_fraction": round(covered / total, 4) if total else None,
        "copy_queues": sorted({r["Queue_Id"] for r in copies}),
        "attention_queues": sorted({r["Queue_Id"] for r in rows
                                    if any(k in r["Kernel_Name"] for k in _ATTN_KERNELS)}),
    }))


def _copy_calibration():
    """One torch copy kernel over 1 GiB: reads 1 GiB, writes 1 GiB."""
    import torch
    n = 1 << 28  # float32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4}), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_lwm7b_fwd_bwd.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_lwm7b.json")
KERNEL_SOURCES = {
    "fwd_bf16": ["blockwise_ring_attention_amd/csrc/fwd_bf16.hip"],
    "bwd_dq": ["blockwise_ring_attention_amd/csrc/bwd_bf16.hip"],
    "bwd_dkv": ["blockwise_ring_attention_amd/csrc/bwd_bf16.hip"],
    "fwd_decode": ["blockwise_ring_attention_amd/csrc/decode_bf16.hip"],
    "ffn_up": ["blockwise_ring_attention_amd/csrc/ffn_bf16.hip"],
    "ffn_down": ["blockwise_ring_attention_amd/csrc/ffn_bf16.hip"],
    "ffn_bwd_gemm": ["blockwise_ring_attention_amd/csrc/ffn_bf16.hip"],
}
COMMON_SOURCE = "blockwise_ring_attention_amd/csrc/ra_common.h"


def _profiled(family, path=TRAFFIC_FILE):
    """The committed counter record of a kernel family (and the file's
    calibration factors), or None when the kernel's source has changed since
    the counters were taken."""
    import hashlib
    try:
        with open(path) as f:
            rec = json.load(f)
        k = rec["kernels"][family]
        h = hashlib.sha256()
        for path in KERNEL_SOURCES[family] + [COMMON_SOURCE]:
            with open(os.path.join(ROOT, path), "rb") as f:
                h.update(f.read())
        if h.hexdigest()[:16] != k["source_sha256_16"]:
            return None
        return rec, k
    except (OSError, KeyError, ValueError):
        return None


def _measured_traffic(family, path=TRAFFIC_FILE):
    """HBM bytes per launch of a kernel family from the committed FETCH_SIZE /
    WRITE_SIZE counter runs (scaled by the copy calibration), or None."""
    p = _profiled(family, path)
    if p is None:
        return None
    rec, k = p
    kib = k["fetch_kib_per_dispatch"] * rec["fetch_factor"] + \
        k["write_kib_per_dispatch"] * rec["write_factor"]
    return int(kib * 1024)


def _measured_mfma_util(family):
    """MFMA busy percentage of a past-block launch (rocprofv3's MfmaUtil:
    SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs), or None."""
    p = _profiled(family)
    return None if p is None else p[1].get("mfma_util_pct")


# State a forked oracle worker inherits (set just before the pool forks).
_ORACLE_POOL_STATE = {}


def _oracle_pool_init():
    """Pool worker: one BLAS thread and one torch thread per process."""
    import torch
    from threadpoolctl import threadpool_limits
    torch.set_num_threads(1)
    _ORACLE_POOL_STATE["limits"] = threadpool_limits(1)


def _oracle_task(task):
    """The fp64 oracle on one slice of the share: head h, query rows
    [r0, r0 + n), against every key block the member sees; forward and, for
    training shares, the gradients.  Returns (unmasked pairs, seconds)."""
    import numpy as np
    import torch

    import oracle
    st = _ORACLE_POOL_STATE
    host, cfg, rank, backward, k_pos = (st["host"], st["cfg"], st["rank"], st["backward"],
                                        st["k_pos"])
    h, r0, n = task
    blocks = sorted(host.kv)
    t0 = time.perf_counter()
    kh = oracle.exact._kv_head(h, cfg.heads, cfg.n_kv_heads)
    k = torch.cat([host.kv[b][0][:, kh:kh + 1] for b in blocks], dim=2)
    v = torch.cat([host.kv[b][1][:, kh:kh + 1] for b in blocks], dim=2)
    rows = np.arange(r0, r0 + n)
    q_pos = oracle.positions(rank, cfg.block_len)[rows]
    q = host.q[:, h:h + 1, rows]
    if backward:
        oracle.attention_grads(q, k, v, host.dout[:, h:h + 1, rows], q_pos, k_pos, cfg.causal)
    else:
        oracle.attention(q, k, v, q_pos, k_pos, cfg.causal)
    dt = time.perf_counter() - t0
    pairs = int(sum(int((k_pos <= p).sum()) if cfg.causal else len(k_pos) for p in q_pos))
    return pairs * cfg.batch, dt


def _cpu_share():
    """CPUs this process may use, capped at 16: the host CPU share of one GPU."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_baseline(host, cfg, rank, backward, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same share,
    timed on the host: a pool of P processes (P = the CPU share, one BLAS
    thread each) works through (head, 256-row tile) slices, the last tiles
    of every head first (rows that see every key block).  One round of P
    slices sizes the sample; then enough rounds for about target_s seconds
    are timed.  Call before anything initialises the GPU: the pool forks."""
    import multiprocessing as mp

    import numpy as np

    import oracle
    L = cfg.block_len
    blocks = sorted(host.kv)
    P = _cpu_share()
    _ORACLE_POOL_STATE.update(host=host, cfg=cfg, rank=rank, backward=backward,
                              k_pos=np.concatenate([oracle.positions(b, L) for b in blocks]))
    tile = 256
    tasks = [(h, r0, min(tile, L - r0)) for r0 in range(((L - 1) // tile) * tile, -1, -tile)
             for h in range(cfg.heads)]
    with mp.get_context("fork").Pool(P, initializer=_oracle_pool_init) as pool:
        t0 = time.perf_counter()
        pool.map(_oracle_task, tasks[:P], chunksize=1)
        t_round = time.perf_counter() - t0
        rounds = max(1, min(len(tasks) // P - 1, int(round(target_s / max(t_round, 1e-3)))))
        todo = tasks[P:P + rounds * P] or tasks[:P]
        t0 = time.perf_counter()
        res = pool.map(_oracle_task, todo, chunksize=1)
        wall = time.perf_counter() - t0
    pairs = sum(r[0] for r in res)
    per_pair = (FWD_FLOPS_PER_PAIR_PER_D + (BWD_FLOPS_PER_PAIR_PER_D if backward else 0))
    flops = per_pair * cfg.head_dim * pairs
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": P, "kind": "oracle",
            "processes": P, "blas_threads_per_process": 1,
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
            "sample": (f"fp64 oracle {'forward + gradients' if backward else 'forward'} of "
                       f"{len(todo)} (head, 256-row tile) slices (the last tiles of each head "
                       f"first) against all {len(_ORACLE_POOL_STATE['k_pos'])} keys, "
                       f"{pairs} unmasked pairs, {wall:.1f} s on {P} processes"),
            "seconds": round(wall, 2)}


def _cpu_model():
    """CPU model from lscpu, else /proc/cpuinfo."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            return next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        return "unknown"


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _decode_bytes(cfg, splits):
    """Algorithmic HBM bytes of one decode step: the split kernel reads q and
    the key/value block once and writes each split's (o, lse) partial; the
    fold reads the partials and the accumulator and writes the accumulator."""
    rows = cfg.batch * cfg.heads * cfg.q_len
    d = cfg.head_dim
    kv = 2 * cfg.batch * cfg.n_kv_heads * cfg.kv_len * d * 2
    part = splits * rows * (d + 1) * 4
    split_kernel = rows * d * 2 + kv + part
    fold = part + 2 * rows * (d + 1) * 4
    return split_kernel, fold


def _decode_cpu_baseline(cfg, q, kvs, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the decode step:
    whole (batch, key/value head) groups, in order, until about target_s."""
    import numpy as np
    import torch

    import oracle

    Lk, G = cfg.kv_len, cfg.heads // cfg.n_kv_heads
    k_pos = np.concatenate([oracle.positions(i, Lk) for i in range(len(kvs))])
    q_pos = oracle.positions(len(kvs), Lk, cfg.q_len)
    done, t0 = 0, time.perf_counter()
    groups = [(b, kh) for b in range(cfg.batch) for kh in range(cfg.n_kv_heads)]
    for b, kh in groups:
        k = torch.cat([kv[0, b:b + 1, kh:kh + 1] for kv in kvs], dim=2)
        v = torch.cat([kv[1, b:b + 1, kh:kh + 1] for kv in kvs], dim=2)
        oracle.attention(q[b:b + 1, kh * G:(kh + 1) * G], k, v, q_pos, k_pos, True)
        done += 1
        if time.perf_counter() - t0 > target_s:
            break
    dt = time.perf_counter() - t0
    frac = done / len(groups)
    split_bytes, _ = _decode_bytes(cfg, 1)
    return {"value": split_bytes * frac / dt / 1e9, "unit": "GB/s", "cores": int(_oracle_threads()),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": (f"fp64 oracle attention of {done} of {len(groups)} (batch, key/value head) "
                       f"groups ({G * cfg.q_len} query rows each against {len(k_pos)} keys), "
                       f"{dt:.1f} s; bytes are the q and key/value bytes of those groups"),
            "seconds": round(dt, 2)}


def _bench_decode(args):
    import torch

    from blockwise_ring_attention_amd import _lib
    from blockwise_ring_attention_amd.configs import DECODE_CONFIGS
    from blockwise_ring_attention_amd.inputs import draw_decode
    from dataclasses import replace

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    _lib.load()
    cfg = replace(DECODE_CONFIGS["decode-lwm7b"], kv_heads=args.kv_heads)
    mha = cfg.n_kv_heads == cfg.heads
    t_gen = time.perf_counter()
    q, kvs = draw_decode(cfg, seed=0)
    dev = torch.device("cuda:0")
    qd = q.to(dev)
    kvd = [kv.to(dev) for kv in kvs]
    o_acc = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse_acc = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    kc = cfg.k_chunk or _lib.ring_attn_decode_chunk(qd, kvd[0])
    S = _lib.ring_attn_decode_splits(qd, kvd[0], kc)
    o_part = torch.empty((S,) + tuple(q.shape), dtype=torch.float32, device=dev)
    lse_part = torch.empty((S,) + tuple(q.shape[:3]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    main_stream = torch.cuda.current_stream()

    def step():
        _lib.ring_attn_init_acc(o_acc, lse_acc)
        for kv in kvd:
            _lib.ring_attn_fwd_decode(qd, kv, kc, o_acc, lse_acc, o_part, lse_part)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.ring_attn_timing_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    w0 = time.perf_counter()
    ev[0].record(main_stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(main_stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) * 1e3 / args.steps
    _lib.ring_attn_timing_enable(False)
    ms_step = ev[0].elapsed_time(ev[args.steps]) / args.steps
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]

    split_bytes, fold_bytes = _decode_bytes(cfg, S)
    nblk = len(kvd)
    gbs = (split_bytes + fold_bytes) * nblk / (ms_step * 1e-3) / 1e9
    per_kernel = {}
    for fam, nbytes in (("fwd_decode", split_bytes), ("decode_fold", fold_bytes)):
        n, tot = _lib.ring_attn_timing_read(fam)
        if n == 0:
            continue
        avg = tot / n
        per_kernel[fam] = {"launches": n, "avg_ms": round(avg, 4),
                           "bytes_per_launch": nbytes,
                           "gbs": round(nbytes / (avg * 1e-3) / 1e9, 1),
                           "frac": round(nbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    dom = "fwd_decode"
    roofline = {"bound": "hbm", "achieved": per_kernel[dom]["gbs"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": per_kernel[dom]["frac"],
                "traffic": (_measured_traffic(dom, DECODE_TRAFFIC_FILE) if mha else None),
                "traffic_unit": "HBM bytes per launch", "kernel": dom}
    result = {
        "metric": "decode-step HBM GB/s (algorithmic bytes: key/value block read once)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"decode-lwm7b: batch {cfg.batch}, {cfg.heads} heads"
                                + (f" ({cfg.n_kv_heads} key/value heads)" if not mha else "")
                                + f", head_dim {cfg.head_dim}, {cfg.q_len} query row(s) "
                                f"against {cfg.kv_len} keys"),
                   "batch": cfg.batch, "heads": cfg.heads, "kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "q_len": cfg.q_len, "kv_len": cfg.kv_len,
                   "blocks": nblk, "k_chunk": kc, "splits": S},
        "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "decode_rows_per_s": round(cfg.batch * cfg.q_len / (ms_step * 1e-3), 1),
        "wall_ms_per_step": round(wall, 4),
        "step_ms_median": round(sorted(step_ms)[len(step_ms) // 2], 4),
        "step_ms_min": round(min(step_ms), 4),
        "kernels": per_kernel,
        "roofline": roofline,
        "input_setup_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _decode_cpu_baseline(cfg, q, kvs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


FFN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ffn_lwm7b.json")


def _ffn_cpu_baseline(x, w1, w2, dout, target_s):
    """The fp64 oracle, as it stands, forward and gradients on a bounded
    sample of the rows (the first n rows, n growing until about target_s)."""
    import oracle

    def run(n):
        t0 = time.perf_counter()
        oracle.feedforward(x[:n], w1, w2)
        oracle.feedforward_grads(x[:n], w1, w2, dout[:n])
        return time.perf_counter() - t0

    n = 8
    dt = run(n)
    while dt < target_s / 4 and n < x.shape[0]:
        n = min(x.shape[0], n * 4)
        dt = run(n)
    flops = 14.0 * n * w1.shape[1] * w1.shape[0]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(_oracle_threads()),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": (f"fp64 oracle feedforward and gradients of the first {n} of {x.shape[0]} "
                       f"rows (d_model {w1.shape[1]}, d_ff {w1.shape[0]}), {dt:.1f} s"),
            "seconds": round(dt, 2)}


def _bench_ffn(args):
    import torch

    from blockwise_ring_attention_amd import _lib
    from blockwise_ring_attention_amd.configs import FFN_CONFIGS
    from blockwise_ring_attention_amd.inputs import draw_ffn, draw_ffn_dout

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    _lib.load()
    cfg = FFN_CONFIGS["ffn-lwm7b"]
    t_gen = time.perf_counter()
    x, w1, w2 = draw_ffn(cfg, seed=0)
    dout = draw_ffn_dout(cfg, seed=0)
    dev = torch.device("cuda:0")
    xd, w1d, w2d, dd = x.to(dev), w1.to(dev), w2.to(dev), dout.to(dev)
    hidden = torch.empty((min(cfg.rows, cfg.chunk_rows), cfg.d_ff), dtype=torch.bfloat16,
                         device=dev)
    out = torch.empty((cfg.rows, cfg.d_model), dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(xd)
    dw1 = torch.zeros((cfg.d_ff, cfg.d_model), dtype=torch.float32, device=dev)
    dw2 = torch.zeros((cfg.d_model, cfg.d_ff), dtype=torch.float32, device=dev)
    work = torch.empty(_lib.ring_ffn_bwd_workspace(cfg.rows, cfg.d_model, cfg.d_ff,
                                                   cfg.chunk_rows), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    main_stream = torch.cuda.current_stream()

    def fwd():
        _lib.ring_ffn_fwd(xd, w1d, w2d, hidden, out, cfg.chunk_rows)

    def bwd():
        _lib.ring_ffn_bwd(xd, w1d, w2d, dd, dx, dw1, dw2, work, cfg.chunk_rows)

    def step():
        fwd()
        bwd()

    def timed(fn, steps, per_step=None):
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        w0 = time.perf_counter()
        ev[0].record(main_stream)
        for i in range(steps):
            fn()
            ev[i + 1].record(main_stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) * 1e3 / steps
        if per_step is not None:
            per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        return ev[0].elapsed_time(ev[steps]) / steps, wall

    for _ in range(args.warmup):
        step()
    _lib.ring_attn_timing_enable(True)
    step_ms = []
    ms_step, wall = timed(step, args.steps, step_ms)
    _lib.ring_attn_timing_enable(False)
    chunks = (cfg.rows + cfg.chunk_rows - 1) // cfg.chunk_rows
    unit = 2.0 * cfg.rows * cfg.d_model * cfg.d_ff     # one product over all rows
    fwd_flops, bwd_flops = 2 * unit, 5 * unit
    tflops = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    # flops per step of each timed family (the backward's products in total)
    fam_flops = {"ffn_up": unit, "ffn_down": unit, "ffn_bwd_gemm": 5 * unit}
    per_kernel = {}
    for fam in ("ffn_up", "ffn_down", "ffn_bwd_gemm", "ffn_bwd_aux"):
        n, tot = _lib.ring_attn_timing_read(fam)
        if n == 0:
            continue
        rec = {"launch_groups": n, "total_ms_per_step": round(tot / args.steps, 4)}
        if fam in fam_flops:
            tf = fam_flops[fam] * args.steps / (tot * 1e-3) / 1e12
            rec.update({"tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
            if fam in ("ffn_up", "ffn_down"):
                rec["avg_ms"] = round(tot / n, 4)
                rec["flops_per_launch"] = unit / chunks
        per_kernel[fam] = rec
    phases = {}
    if not args.no_phases:
        ms_f, _ = timed(fwd, args.steps)
        ms_b, _ = timed(bwd, args.steps)
        for name, ms, fl in (("fwd", ms_f, fwd_flops), ("bwd", ms_b, bwd_flops)):
            tf = fl / (ms * 1e-3) / 1e12
            phases[name] = {"ms": round(ms, 3), "tflops": round(tf, 1),
                            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    flops_fams = [f for f in per_kernel if "tflops" in per_kernel[f]]
    dom = max(flops_fams, key=lambda f: per_kernel[f]["total_ms_per_step"])
    roofline = {"bound": "mfma", "achieved": per_kernel[dom]["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": per_kernel[dom]["frac"],
                "traffic": _measured_traffic(dom, FFN_TRAFFIC_FILE),
                "traffic_unit": "HBM bytes per product launch", "kernel": dom}
    result = {
        "metric": ("blockwise feedforward training-step TFLOP/s (fwd 4 + bwd 10 "
                   "·rows·d_model·d_ff); % of bf16 MFMA peak"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"ffn-lwm7b fwd+bwd: {cfg.rows} rows, d_model {cfg.d_model}, "
                                f"d_ff {cfg.d_ff}, GELU, {cfg.chunk_rows} rows per chunk"),
                   "rows": cfg.rows, "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "chunk_rows": cfg.chunk_rows},
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "wall_ms_per_step": round(wall, 4),
        "step_ms_median": round(sorted(step_ms)[len(step_ms) // 2], 4),
        "step_ms_min": round(min(step_ms), 4),
        "phases": phases,
        "kernels": per_kernel,
        "roofline": roofline,
        "input_setup_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _ffn_cpu_baseline(x, w1, w2, dout, args.cpu_seconds)
    print(json.dumps(result), flush=True)


# Attention workloads that --config selects (the configs of the share's
# parity tests): 3 (default) is the 16384-query causal share with its
# backward; 2 and 5 are forward-only shares; 4 is the training share.
SHARE_WORKLOADS = {
    2: "non-causal share fwd: batch 2, 16 heads, head_dim 128, ring 8, 4096 local queries x 32768 keys",
    3: "lwm7b-causal-ring-share fwd+bwd: batch 1, 32 heads, head_dim 128, ring 8, rank 7, "
       "16384 local queries x 131072 keys",
    4: "training share fwd+bwd: batch 1, 32 heads, head_dim 128, ring 4, rank 3, "
       "8192 local queries x 32768 keys",
    5: "million-token ring share fwd: batch 1, 32 heads, head_dim 128, ring 64, rank 31, "
       "16384 local queries x 524288 keys (adversarial scores)",
}


def main():
    args = _parse()
    if args.trace_overlap:
        _trace_overlap(args.trace_overlap)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one ring member's share on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported: the multi-GPU ring is not part of this "
              "build.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        _copy_calibration()
        return
    if args.decode:
        _bench_decode(args)
        return
    if args.ffn:
        _bench_ffn(args)
        return
    if args.config not in SHARE_WORKLOADS:
        print(f"--config {args.config}: choose one of {sorted(SHARE_WORKLOADS)}", file=sys.stderr)
        sys.exit(2)

    import torch

    from blockwise_ring_attention_amd import share
    from blockwise_ring_attention_amd.configs import CONFIGS, scaled

    backward = args.config in (3, 4)
    cfg = scaled(CONFIGS[args.config], backward=backward, kv_heads=args.kv_heads)
    mha = cfg.n_kv_heads == cfg.heads
    rank = cfg.ranks[0]
    t_gen = time.perf_counter()
    host = share.make_host_share(cfg, rank, seed=0, backward=backward)
    t_gen = time.perf_counter() - t_gen
    # The oracle's pool forks, so it runs before anything touches the GPU.
    cpu = None if args.no_cpu_baseline else _cpu_baseline(host, cfg, rank, backward,
                                                          args.cpu_seconds)

    from blockwise_ring_attention_amd import _lib
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    _lib.load()
    t_up = time.perf_counter()
    dev = share.upload(host)
    torch.cuda.synchronize()
    t_gen += time.perf_counter() - t_up
    main_stream = torch.cuda.current_stream()
    side = share.side_stream_for(dev.q.device)

    def fwd():
        share.forward(dev, side_stream=side)
        return share.finalize(dev)

    def bwd():
        share.backward(dev, side_stream=side)

    def step():
        fwd()
        if backward:
            bwd()

    def timed(fn, steps, per_step=None):
        """Mean ms per step between two events around all steps (and, if
        per_step is a list, each step's own ms appended to it)."""
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        w0 = time.perf_counter()
        ev[0].record(main_stream)
        for i in range(steps):
            fn()
            ev[i + 1].record(main_stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) * 1e3 / steps
        if per_step is not None:
            per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        return ev[0].elapsed_time(ev[steps]) / steps, wall

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.ring_attn_timing_enable(True)
    step_ms = []
    ms_step, wall_step = timed(step, args.steps, step_ms)
    _lib.ring_attn_timing_enable(False)
    kernels = {}
    for fam in ("fwd_bf16", "bwd_dq", "bwd_dkv") if backward else ("fwd_bf16",):
        n, tot = _lib.ring_attn_timing_read(fam)
        kernels[fam] = {"launches": n, "total_ms": tot}

    pairs = cfg.pairs(rank)
    d = cfg.head_dim
    fwd_flops = FWD_FLOPS_PER_PAIR_PER_D * d * pairs
    bwd_flops = BWD_FLOPS_PER_PAIR_PER_D * d * pairs if backward else 0
    tflops = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12

    phases = {}
    if backward and not args.no_phases:
        ms_fwd, _ = timed(fwd, args.steps)
        ms_bwd, _ = timed(bwd, args.steps)
        for name, ms, fl in (("fwd", ms_fwd, fwd_flops), ("bwd", ms_bwd, bwd_flops)):
            tf = fl / (ms * 1e-3) / 1e12
            phases[name] = {"ms": round(ms, 3), "tflops": round(tf, 1),
                            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}

    # Roofline of the kernel family that takes the most time in the step.
    # The committed counters were taken on the default workload only.
    counters = mha and args.config == 3
    per_kernel = {}
    for fam, rec in kernels.items():
        if rec["launches"] == 0:
            continue
        flops = KERNEL_FLOPS_PER_PAIR_PER_D[fam] * d * pairs * args.steps
        avg_ms = rec["total_ms"] / rec["launches"]
        achieved = flops / (rec["total_ms"] * 1e-3) / 1e12
        per_kernel[fam] = {"launches": rec["launches"], "avg_ms": round(avg_ms, 4),
                           "total_ms_per_step": round(rec["total_ms"] / args.steps, 3),
                           "tflops": round(achieved, 1),
                           "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                           "mfma_busy_pct_counter": _measured_mfma_util(fam) if counters else None}
    dom = max(per_kernel, key=lambda f: per_kernel[f]["total_ms_per_step"])
    roofline = {"bound": "mfma", "achieved": per_kernel[dom]["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": per_kernel[dom]["frac"],
                "traffic": _measured_traffic(dom) if counters else None,
                "traffic_unit": "HBM bytes per launch",
                "mfma_busy_pct_counter": _measured_mfma_util(dom) if counters else None,
                "kernel": dom}

    workload = SHARE_WORKLOADS[args.config]
    if cfg.n_kv_heads != cfg.heads:
        workload += f", {cfg.n_kv_heads} shared key/value heads"
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "config": args.config,
                   "pass": "fwd+bwd" if backward else "fwd",
                   "batch": cfg.batch, "heads": cfg.heads, "kv_heads": cfg.n_kv_heads,
                   "head_dim": d,
                   "ring_size": cfg.ring_size, "rank": rank, "local_queries": cfg.block_len,
                   "keys": cfg.block_len * len(cfg.kv_blocks_seen(rank)), "causal": cfg.causal,
                   "q_chunk": cfg.q_chunk, "k_chunk": cfg.k_chunk,
                   "unmasked_pairs": pairs},
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "wall_ms_per_step": round(wall_step, 3),
        "step_ms_median": round(sorted(step_ms)[len(step_ms) // 2], 3),
        "step_ms_min": round(min(step_ms), 3),
        "phases": phases,
        "kernels": per_kernel,
        "roofline": roofline,
        "input_setup_s": round(t_gen, 1),
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
