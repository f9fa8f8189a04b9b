"""ctypes binding of ``libringattn.so`` (declared in ``include/ring_attn.h``).

Argument marshalling only: every function takes torch CUDA tensors, checks
that they are contiguous device tensors of the dtype the C ABI expects,
passes their device pointers, dims and the current HIP stream, and turns a
negative return code into ``RingAttnError``.  All arithmetic happens in the
HIP kernels.  There is no fallback: if the library is missing, loading it
raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libringattn.so")

RA_BF16, RA_FP32 = 0, 1
RA_EMU_OVERLAP, RA_EMU_SERIALIZE, RA_EMU_UNSAFE = 0, 1, 2
# RA_DECODE_SCRATCH_BYTES: size of the library's decode scratch array
DECODE_SCRATCH_BYTES = 16 << 20
_ERR_NAMES = {-1: "invalid argument", -2: "unsupported", -3: "HIP error"}


class RingAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {message}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("kv_heads", ctypes.c_int32)]


_lib = None
_lock = threading.Lock()
_vp = ctypes.c_void_p
_i = ctypes.c_int
_SIGS = {
    "ring_attn_version": ([], _i),
    "ring_attn_last_error": ([], ctypes.c_char_p),
    "ring_attn_init_acc": ([_vp, _vp, ctypes.POINTER(Dims), _vp], _i),
    "ring_attn_fwd": ([_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, ctypes.POINTER(Dims), _vp], _i),
    "ring_attn_combine": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Dims), _vp], _i),
    "ring_attn_finalize": ([_vp, _vp, _i, ctypes.POINTER(Dims), _vp], _i),
    "ring_attn_bwd_prep": ([_vp, _vp, _vp, ctypes.POINTER(Dims), _vp], _i),
    "ring_attn_bwd": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp,
                       ctypes.POINTER(Dims), _vp], _i),
    "ring_attn_bwd_workspace": ([ctypes.POINTER(Dims)], ctypes.c_int64),
    "ring_attn_bwd_ws": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp,
                          ctypes.c_int64, ctypes.POINTER(Dims), _vp], _i),
    "ring_emu_fwd": ([_vp, ctypes.POINTER(_vp), _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp,
                      ctypes.POINTER(Dims), ctypes.POINTER(ctypes.c_int32), _i, _vp, _vp], _i),
    "ring_emu_bwd": ([_vp, ctypes.POINTER(_vp), _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_vp),
                      _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, ctypes.c_int64, ctypes.POINTER(Dims),
                      ctypes.POINTER(ctypes.c_int32), _i, _vp, _vp], _i),
    "ring_attn_decode_chunk": ([ctypes.POINTER(Dims)], _i),
    "ring_attn_decode_splits": ([ctypes.POINTER(Dims), _i], _i),
    "ring_attn_fwd_decode": ([_vp, _vp, _i, _vp, _vp, _vp, _vp, ctypes.POINTER(Dims), _vp], _i),
    "ring_attn_fwd_decode_noalloc": ([_vp, _vp, _i, _vp, _vp, ctypes.POINTER(Dims), _vp], _i),
    "ring_ffn_fwd": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_int64, _i, _i, _i, _vp], _i),
    "ring_ffn_bwd_workspace": ([ctypes.c_int64, _i, _i, _i], ctypes.c_int64),
    "ring_ffn_bwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64, _i, _i,
                      _i, _vp], _i),
    "ring_attn_timing_enable": ([_i], _i),
    "ring_attn_timing_read": ([ctypes.c_char_p, ctypes.POINTER(_i), ctypes.POINTER(ctypes.c_double)], _i),
}
EXPORTS = tuple(_SIGS)


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise ImportError(
                f"{p} not found: build the HIP library first "
                "(python -m blockwise_ring_attention_amd.build)")
        lib = ctypes.CDLL(p)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        if path is None:
            _lib = lib
        return lib


def last_error() -> str:
    return load().ring_attn_last_error().decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise RingAttnError(rc, last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return _vp(t.data_ptr()) if t.numel() else None


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return _vp(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def dims(q: torch.Tensor, kv_len: int, scale: float = 0.0, kv_heads: int = 0) -> Dims:
    """Dims of a call from the query tensor [B, H, Lq, d], the block length
    and the number of key/value heads (0: one per query head)."""
    B, H, Lq, d = q.shape
    return Dims(B, H, Lq, kv_len, d, _dtype_code(q), float(scale), int(kv_heads))


def ring_attn_init_acc(o_acc, lse_acc, scale=0.0, stream=None):
    _need(o_acc, torch.float32, "o_acc")
    _need(lse_acc, torch.float32, "lse_acc")
    B, H, Lq, d = o_acc.shape
    dm = Dims(B, H, Lq, 0, d, RA_FP32, float(scale))
    _check(load().ring_attn_init_acc(_ptr(o_acc), _ptr(lse_acc), ctypes.byref(dm), _stream(stream)))


def ring_attn_fwd(q, kv_block, ring_rank, ring_step, ring_size, causal, q_chunk, k_chunk,
                  o_acc, lse_acc, scale=0.0, stream=None):
    _need(kv_block, q.dtype, "kv_block")
    _need(o_acc, torch.float32, "o_acc")
    _need(lse_acc, torch.float32, "lse_acc")
    dm = dims(q, kv_block.shape[3], scale, kv_block.shape[2])
    _check(load().ring_attn_fwd(_ptr(q), _ptr(kv_block), ring_rank, ring_step, ring_size,
                                int(bool(causal)), q_chunk, k_chunk, _ptr(o_acc), _ptr(lse_acc),
                                ctypes.byref(dm), _stream(stream)))


def _decode_dims(q, kv_block, scale):
    if kv_block.dim() != 5 or kv_block.shape[0] != 2:
        raise ValueError("kv_block must be [2, B, Hkv, Lk, d]")
    return dims(q, kv_block.shape[3], scale, kv_block.shape[2])


def ring_attn_decode_chunk(q, kv_block, scale=0.0) -> int:
    """Keys per split that spread a decode step of these shapes over the chip."""
    dm = _decode_dims(q, kv_block, scale)
    rc = load().ring_attn_decode_chunk(ctypes.byref(dm))
    _check(min(rc, 0))
    return rc


def ring_attn_decode_splits(q, kv_block, k_chunk, scale=0.0) -> int:
    """Number of key splits S = ceil(Lk / k_chunk) (rows of o_part / lse_part)."""
    dm = _decode_dims(q, kv_block, scale)
    rc = load().ring_attn_decode_splits(ctypes.byref(dm), int(k_chunk))
    _check(min(rc, 0))
    return rc


def ring_attn_fwd_decode(q, kv_block, k_chunk, o_acc, lse_acc, o_part, lse_part, scale=0.0,
                         stream=None):
    """Decode-shaped step: folds attention(q, kv_block) (no mask) into
    (o_acc, lse_acc); o_part [S, B, H, Lq, d] / lse_part [S, B, H, Lq] hold
    the key splits' partials, S from ring_attn_decode_splits."""
    _need(kv_block, q.dtype, "kv_block")
    for t, n in ((o_acc, "o_acc"), (lse_acc, "lse_acc"), (o_part, "o_part"),
                 (lse_part, "lse_part")):
        _need(t, torch.float32, n)
    dm = _decode_dims(q, kv_block, scale)
    S = ring_attn_decode_splits(q, kv_block, k_chunk, scale)
    if tuple(o_acc.shape) != tuple(q.shape) or tuple(lse_acc.shape) != tuple(q.shape[:3]):
        raise ValueError("o_acc / lse_acc do not match q")
    if o_part.numel() < S * q.numel() or lse_part.numel() < S * lse_acc.numel():
        raise ValueError(f"o_part / lse_part hold fewer than {S} partials")
    _check(load().ring_attn_fwd_decode(_ptr(q), _ptr(kv_block), int(k_chunk), _ptr(o_acc),
                                       _ptr(lse_acc), _ptr(o_part), _ptr(lse_part),
                                       ctypes.byref(dm), _stream(stream)))


def ring_attn_fwd_decode_noalloc(q, kv_block, k_chunk, o_acc, lse_acc, scale=0.0,
                                 stream=None):
    """ring_attn_fwd_decode with the split partials in the library's own
    device scratch array (nothing allocated; calls on one GPU must not
    overlap in time)."""
    _need(kv_block, q.dtype, "kv_block")
    for t, n in ((o_acc, "o_acc"), (lse_acc, "lse_acc")):
        _need(t, torch.float32, n)
    if tuple(o_acc.shape) != tuple(q.shape) or tuple(lse_acc.shape) != tuple(q.shape[:3]):
        raise ValueError("o_acc / lse_acc do not match q")
    dm = _decode_dims(q, kv_block, scale)
    _check(load().ring_attn_fwd_decode_noalloc(_ptr(q), _ptr(kv_block), int(k_chunk),
                                               _ptr(o_acc), _ptr(lse_acc), ctypes.byref(dm),
                                               _stream(stream)))


def ring_ffn_fwd(x, w1, w2, hidden, out, chunk_rows, stream=None):
    """Blockwise feedforward out = GELU(x w1^T) w2^T over x [rows, d_model],
    chunk_rows rows at a time through the caller's hidden [>= min(rows,
    chunk_rows), d_ff] workspace; all bf16."""
    for t, n in ((x, "x"), (w1, "w1"), (w2, "w2"), (hidden, "hidden"), (out, "out")):
        _need(t, torch.bfloat16, n)
    rows, d_model = x.shape
    d_ff = w1.shape[0]
    if tuple(w1.shape) != (d_ff, d_model) or tuple(w2.shape) != (d_model, d_ff):
        raise ValueError("w1 must be [d_ff, d_model] and w2 [d_model, d_ff]")
    if tuple(out.shape) != (rows, d_model):
        raise ValueError("out must be [rows, d_model]")
    if hidden.numel() < min(rows, max(int(chunk_rows), 1)) * d_ff:
        raise ValueError("hidden holds fewer than min(rows, chunk_rows) x d_ff elements")
    _check(load().ring_ffn_fwd(_ptr(x), _ptr(w1), _ptr(w2), _ptr(hidden), _ptr(out), rows,
                               d_model, d_ff, int(chunk_rows), _stream(stream)))


def ring_ffn_bwd_workspace(rows, d_model, d_ff, chunk_rows) -> int:
    """Bytes of device workspace ring_ffn_bwd needs for these shapes."""
    n = load().ring_ffn_bwd_workspace(int(rows), int(d_model), int(d_ff), int(chunk_rows))
    _check(int(min(n, 0)))
    return int(n)


def ring_ffn_bwd(x, w1, w2, dout, dx, dw1, dw2, work, chunk_rows, stream=None):
    """Backward of ring_ffn_fwd: dx [rows, d_model] bf16 is written, dw1
    [d_ff, d_model] and dw2 [d_model, d_ff] fp32 are accumulated; work is a
    uint8 device tensor of at least ring_ffn_bwd_workspace(...) bytes."""
    for t, n in ((x, "x"), (w1, "w1"), (w2, "w2"), (dout, "dout"), (dx, "dx")):
        _need(t, torch.bfloat16, n)
    _need(dw1, torch.float32, "dw1")
    _need(dw2, torch.float32, "dw2")
    rows, d_model = x.shape
    d_ff = w1.shape[0]
    if tuple(w1.shape) != (d_ff, d_model) or tuple(w2.shape) != (d_model, d_ff):
        raise ValueError("w1 must be [d_ff, d_model] and w2 [d_model, d_ff]")
    if tuple(dout.shape) != (rows, d_model) or tuple(dx.shape) != (rows, d_model):
        raise ValueError("dout and dx must be [rows, d_model]")
    if tuple(dw1.shape) != (d_ff, d_model) or tuple(dw2.shape) != (d_model, d_ff):
        raise ValueError("dw1 must be [d_ff, d_model] and dw2 [d_model, d_ff]")
    nbytes = work.numel() * work.element_size()
    _check(load().ring_ffn_bwd(_ptr(x), _ptr(w1), _ptr(w2), _ptr(dout), _ptr(dx), _ptr(dw1),
                               _ptr(dw2), _ptr(work), nbytes, rows, d_model, d_ff,
                               int(chunk_rows), _stream(stream)))


def ring_attn_combine(o_a, lse_a, o_b, lse_b, stream=None):
    for t, n in ((o_a, "o_a"), (lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b")):
        _need(t, torch.float32, n)
    B, H, Lq, d = o_a.shape
    dm = Dims(B, H, Lq, 0, d, RA_FP32, 0.0)
    _check(load().ring_attn_combine(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b),
                                    ctypes.byref(dm), _stream(stream)))


def ring_attn_finalize(acc, out, stream=None):
    _need(acc, torch.float32, "acc")
    B, H, Lq, d = acc.shape
    dm = Dims(B, H, Lq, 0, d, RA_FP32, 0.0)
    _check(load().ring_attn_finalize(_ptr(acc), _ptr(out), _dtype_code(out), ctypes.byref(dm),
                                     _stream(stream)))


def ring_attn_bwd_prep(o, dout, delta, stream=None):
    _need(o, torch.float32, "o")
    _need(delta, torch.float32, "delta")
    dm = dims(dout, 0)
    _check(load().ring_attn_bwd_prep(_ptr(o), _ptr(dout), _ptr(delta), ctypes.byref(dm),
                                     _stream(stream)))


def ring_attn_bwd(q, kv_block, dout, lse, delta, ring_rank, ring_step, ring_size, causal,
                  q_chunk, k_chunk, dq_acc, dkv_io, scale=0.0, stream=None):
    _need(kv_block, q.dtype, "kv_block")
    _need(dout, q.dtype, "dout")
    for t, n in ((lse, "lse"), (delta, "delta"), (dq_acc, "dq_acc"), (dkv_io, "dkv_io")):
        _need(t, torch.float32, n)
    dm = dims(q, kv_block.shape[3], scale, kv_block.shape[2])
    _check(load().ring_attn_bwd(_ptr(q), _ptr(kv_block), _ptr(dout), _ptr(lse), _ptr(delta),
                                ring_rank, ring_step, ring_size, int(bool(causal)), q_chunk,
                                k_chunk, _ptr(dq_acc), _ptr(dkv_io), ctypes.byref(dm),
                                _stream(stream)))


def ring_attn_bwd_workspace(q, kv_block, scale=0.0) -> int:
    """Bytes of workspace ring_attn_bwd_ws uses for these shapes (0: none)."""
    dm = dims(q, kv_block.shape[3], scale, kv_block.shape[2])
    n = load().ring_attn_bwd_workspace(ctypes.byref(dm))
    _check(int(min(n, 0)))
    return int(n)


def ring_attn_bwd_ws(q, kv_block, dout, lse, delta, ring_rank, ring_step, ring_size, causal,
                     q_chunk, k_chunk, dq_acc, dkv_io, work, scale=0.0, stream=None):
    """ring_attn_bwd with a device workspace (a tensor, or None for none) that
    lets the query heads sharing a key/value head run side by side."""
    _need(kv_block, q.dtype, "kv_block")
    _need(dout, q.dtype, "dout")
    for t, n in ((lse, "lse"), (delta, "delta"), (dq_acc, "dq_acc"), (dkv_io, "dkv_io")):
        _need(t, torch.float32, n)
    nbytes = 0
    if work is not None:
        if not work.is_contiguous():
            raise ValueError("work must be contiguous")
        nbytes = work.numel() * work.element_size()
    dm = dims(q, kv_block.shape[3], scale, kv_block.shape[2])
    _check(load().ring_attn_bwd_ws(_ptr(q), _ptr(kv_block), _ptr(dout), _ptr(lse), _ptr(delta),
                                   ring_rank, ring_step, ring_size, int(bool(causal)), q_chunk,
                                   k_chunk, _ptr(dq_acc), _ptr(dkv_io),
                                   _ptr(work) if work is not None else None, nbytes,
                                   ctypes.byref(dm), _stream(stream)))


def _ptr_array(ts: Sequence[Optional[torch.Tensor]]):
    arr = (_vp * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = t.data_ptr() if t is not None else None
    return arr


def _order_array(order):
    if order is None:
        return None
    arr = (ctypes.c_int32 * len(order))(*[int(x) for x in order])
    return arr


def _emu_mode(serialize, unsafe):
    if serialize and unsafe:
        raise ValueError("serialize and unsafe exclude each other")
    return RA_EMU_SERIALIZE if serialize else (RA_EMU_UNSAFE if unsafe else RA_EMU_OVERLAP)


def ring_emu_fwd(q, kv_pool, slots, ring_rank, ring_size, causal, q_chunk, k_chunk, o_acc,
                 lse_acc, scale=0.0, order=None, serialize=False, main_stream=None,
                 side_stream=None, unsafe=False):
    """kv_pool: list of ring_size packed blocks (None where never needed);
    slots: two receive buffers shaped like one block."""
    if len(kv_pool) != ring_size:
        raise ValueError("kv_pool must have ring_size entries")
    ref = next(t for t in kv_pool if t is not None)
    dm = dims(q, ref.shape[3], scale, ref.shape[2])
    main = main_stream if main_stream is not None else torch.cuda.current_stream()
    side = side_stream if side_stream is not None else main
    _check(load().ring_emu_fwd(_ptr(q), _ptr_array(kv_pool), _ptr(slots[0]), _ptr(slots[1]),
                               ring_rank, ring_size, int(bool(causal)), q_chunk, k_chunk,
                               _ptr(o_acc), _ptr(lse_acc), ctypes.byref(dm), _order_array(order),
                               _emu_mode(serialize, unsafe),
                               _vp(main.cuda_stream), _vp(side.cuda_stream)))


def ring_emu_bwd(q, kv_pool, slots, dout, lse, delta, dkv_pool, dkv_slots, ring_rank, ring_size,
                 causal, q_chunk, k_chunk, dq_acc, scale=0.0, order=None, serialize=False,
                 main_stream=None, side_stream=None, work=None, unsafe=False):
    """work: optional device workspace of ring_attn_bwd_workspace bytes."""
    if len(kv_pool) != ring_size or len(dkv_pool) != ring_size:
        raise ValueError("pools must have ring_size entries")
    ref = next(t for t in kv_pool if t is not None)
    dm = dims(q, ref.shape[3], scale, ref.shape[2])
    main = main_stream if main_stream is not None else torch.cuda.current_stream()
    side = side_stream if side_stream is not None else main
    _check(load().ring_emu_bwd(_ptr(q), _ptr_array(kv_pool), _ptr(slots[0]), _ptr(slots[1]),
                               _ptr(dout), _ptr(lse), _ptr(delta), _ptr_array(dkv_pool),
                               _ptr(dkv_slots[0]), _ptr(dkv_slots[1]), ring_rank, ring_size,
                               int(bool(causal)), q_chunk, k_chunk, _ptr(dq_acc),
                               _ptr(work) if work is not None else None,
                               work.numel() * work.element_size() if work is not None else 0,
                               ctypes.byref(dm), _order_array(order),
                               _emu_mode(serialize, unsafe),
                               _vp(main.cuda_stream), _vp(side.cuda_stream)))


def ring_attn_timing_enable(on: bool = True) -> None:
    _check(load().ring_attn_timing_enable(int(bool(on))))


def ring_attn_timing_read(name: str):
    """(launches, total_ms) of one kernel family since timing was enabled."""
    n = _i(0)
    ms = ctypes.c_double(0.0)
    _check(load().ring_attn_timing_read(name.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value
