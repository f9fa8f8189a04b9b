"""The C ABI library loads, exports every function ``include/ring_attn.h``
declares, and rejects invalid arguments on the host (no GPU needed: every
case here fails validation before anything is enqueued)."""
import ctypes
import os
import re

import pytest

from blockwise_ring_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ring_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("HIP library not built")
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("ring_attn_fwd", "ring_attn_combine", "ring_attn_bwd", "ring_attn_bwd_prep",
              "ring_attn_finalize", "ring_attn_init_acc", "ring_attn_last_error",
              "ring_attn_version", "ring_emu_fwd", "ring_emu_bwd", "ring_attn_fwd_decode",
              "ring_attn_decode_chunk", "ring_attn_decode_splits", "ring_ffn_fwd",
              "ring_attn_fwd_decode_noalloc", "ring_attn_bwd_ws", "ring_attn_bwd_workspace",
              "ring_ffn_bwd", "ring_ffn_bwd_workspace"):
        assert n in names
    assert sorted(_lib.EXPORTS) == names, "binding and header disagree"


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.ring_attn_version() == 204
    assert lib.ring_attn_last_error() == b""


def _dims(**kw):
    base = dict(batch=1, heads=2, q_len=64, kv_len=64, head_dim=128, dtype=0, scale=0.0,
                kv_heads=0)
    base.update(kw)
    return _lib.Dims(*base.values())


FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x100000)


def _fwd(lib, dims, rank=0, step=0, size=1, causal=1, qc=64, kc=64, q=FAKE, kv=FAKE2,
         o=ctypes.c_void_p(0x10000000), lse=ctypes.c_void_p(0x20000000)):
    return lib.ring_attn_fwd(q, kv, rank, step, size, causal, qc, kc, o, lse,
                             ctypes.byref(dims) if dims is not None else None, None)


@pytest.mark.parametrize("case,code", [
    (dict(dims=None), -1),
    (dict(rank=2, size=2), -1),
    (dict(rank=-1, size=2), -1),
    (dict(step=3, size=3), -1),
    (dict(size=0), -1),
    (dict(qc=0), -1),
    (dict(kc=-4), -1),
    (dict(q=None), -1),
    (dict(o=ctypes.c_void_p(0x1000)), -1),             # o_acc aliases q
])
def test_invalid_arguments_rejected(lib, case, code):
    dims = case.pop("dims", _dims())
    assert _fwd(lib, dims, **case) == code
    assert lib.ring_attn_last_error() != b""


def test_unsupported_and_invalid_dims(lib):
    assert _fwd(lib, _dims(head_dim=96)) == -2
    assert _fwd(lib, _dims(dtype=7)) == -2
    assert _fwd(lib, _dims(batch=-1)) == -1
    assert _fwd(lib, _dims(q_len=64, kv_len=32)) == -1           # causal needs equal blocks
    assert _fwd(lib, _dims(scale=float("inf"))) == -1
    assert _fwd(lib, _dims(scale=-0.5)) == -1
    assert _fwd(lib, _dims(heads=4, kv_heads=3)) == -1             # must divide heads
    assert _fwd(lib, _dims(heads=4, kv_heads=8)) == -1
    assert _fwd(lib, _dims(heads=4, kv_heads=-2)) == -1
    # the backward is bf16-only
    d = _dims(dtype=1)
    assert lib.ring_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 1, 1, 64, 64, FAKE, FAKE,
                             ctypes.byref(d), None) == -2
    assert b"bf16" in lib.ring_attn_last_error()


def _bwd_ws(lib, dims, work, nbytes, **kw):
    p = dict(q=1 << 40, kv=2 << 40, do=3 << 40, lse=4 << 40, delta=5 << 40, dq=6 << 40,
             dkv=7 << 40)
    p.update(kw)
    v = {k: ctypes.c_void_p(x) if x is not None else None for k, x in p.items()}
    return lib.ring_attn_bwd_ws(v["q"], v["kv"], v["do"], v["lse"], v["delta"], 0, 0, 1, 1,
                                256, 64, v["dq"], v["dkv"],
                                ctypes.c_void_p(work) if work is not None else None, nbytes,
                                ctypes.byref(dims) if dims is not None else None, None)


def test_bwd_workspace_planning(lib):
    """Shared key/value heads run enough query heads side by side for about
    one workgroup (128 keys) per compute unit, never more than the group."""
    def ws(**kw):
        return lib.ring_attn_bwd_workspace(ctypes.byref(_dims(**kw)))
    copy = lambda b, hkv, lk, d: 2 * b * hkv * lk * d * 4
    assert ws(heads=32, q_len=16384, kv_len=16384) == 0                 # one kv head each
    assert ws(heads=32, kv_heads=8, q_len=16384, kv_len=16384) == 0     # 1024 workgroups
    # MQA: 128 workgroups, two heads side by side, one copy
    assert ws(heads=32, kv_heads=1, q_len=16384, kv_len=16384) == copy(1, 1, 16384, 128)
    # 16 workgroups -> 16 side by side, capped at the group of 8
    assert ws(heads=8, kv_heads=1, q_len=2048, kv_len=2048) == 7 * copy(1, 1, 2048, 128)
    assert ws(heads=32, kv_heads=2, q_len=4096, kv_len=4096, head_dim=64) == \
        3 * copy(1, 2, 4096, 64)                                          # 64 wgs -> 4 side by side
    assert lib.ring_attn_bwd_workspace(None) == -1
    assert lib.ring_attn_bwd_workspace(ctypes.byref(_dims(head_dim=96))) == -2


def test_bwd_ws_rejects_invalid(lib):
    mqa = _dims(heads=32, kv_heads=1, q_len=16384, kv_len=16384)
    need = lib.ring_attn_bwd_workspace(ctypes.byref(mqa))
    far = 8 << 40
    assert _bwd_ws(lib, None, far, need) == -1
    assert _bwd_ws(lib, mqa, far, -1) == -1
    assert _bwd_ws(lib, mqa, None, need) == -1
    assert b"NULL workspace" in lib.ring_attn_last_error()
    assert _bwd_ws(lib, mqa, far + 4, need) == -1
    assert b"aligned" in lib.ring_attn_last_error()
    assert _bwd_ws(lib, mqa, (7 << 40) + 4096, need) == -1             # overlaps dkv_io
    assert b"workspace overlaps" in lib.ring_attn_last_error()
    assert _bwd_ws(lib, mqa, 1 << 40, need) == -1                      # overlaps q
    assert _bwd_ws(lib, _dims(dtype=1), far, need) == -2
    assert _bwd_ws(lib, mqa, far, need, q=None) == -1
    # nothing to compute: no pointer is touched
    nul = dict(q=None, kv=None, do=None, lse=None, delta=None, dq=None, dkv=None)
    assert _bwd_ws(lib, _dims(heads=32, kv_heads=1, q_len=0, kv_len=0), None, 0, **nul) == 0


def test_empty_problems_are_no_ops(lib):
    # nothing to compute: succeeds without touching a pointer or the GPU
    assert _fwd(lib, _dims(q_len=0, kv_len=0), q=None, kv=None, o=None, lse=None) == 0
    assert _fwd(lib, _dims(batch=0), q=None, kv=None, o=None, lse=None) == 0
    d = _dims(heads=0)
    assert lib.ring_attn_combine(None, None, None, None, ctypes.byref(d), None) == 0


def _decode(lib, dims, kc=64, q=FAKE, kv=FAKE2, o=ctypes.c_void_p(0x10000000),
            lse=ctypes.c_void_p(0x20000000), op=ctypes.c_void_p(0x30000000),
            lp=ctypes.c_void_p(0x40000000)):
    return lib.ring_attn_fwd_decode(q, kv, kc, o, lse, op, lp,
                                    ctypes.byref(dims) if dims is not None else None, None)


def test_decode_rejects_invalid_and_unsupported(lib):
    d1 = _dims(q_len=1, kv_len=4096)
    assert _decode(lib, None) == -1
    assert _decode(lib, _dims(q_len=1, dtype=1)) == -2                 # bf16 only
    assert _decode(lib, _dims(heads=8, kv_heads=1, q_len=9)) == -2      # 72 rows per group
    assert _decode(lib, _dims(heads=2, q_len=65)) == -2
    assert _decode(lib, d1, kc=0) == -1
    assert _decode(lib, d1, kc=-5) == -1
    assert _decode(lib, d1, op=None) == -1
    assert _decode(lib, d1, lp=None) == -1
    assert _decode(lib, d1, q=None) == -1
    assert _decode(lib, _dims(q_len=1, kv_len=70000), kc=1) == -1      # 70000 splits
    # o_part [S, 1, 2, 1, 128] fp32 with S = 64 spans 64 KiB from 0x30000000
    assert _decode(lib, d1, lp=ctypes.c_void_p(0x30000000 + 60000)) == -1  # parts overlap
    assert _decode(lib, d1, op=ctypes.c_void_p(0x10000000 - 1024)) == -1  # overlaps o_acc
    assert _decode(lib, d1, lp=ctypes.c_void_p(0x1000 + 64)) == -1       # overlaps q
    assert b"rows per key/value head group" in _decode_msg(lib, _dims(heads=4, kv_heads=1,
                                                                      q_len=17))


def _decode_msg(lib, dims):
    assert _decode(lib, dims) != 0
    return lib.ring_attn_last_error()


def test_decode_empty_calls_are_no_ops(lib):
    nul = dict(q=None, kv=None, o=None, lse=None, op=None, lp=None)
    assert _decode(lib, _dims(q_len=0), **nul) == 0
    assert _decode(lib, _dims(batch=0, q_len=1), **nul) == 0
    assert _decode(lib, _dims(heads=0, q_len=1), **nul) == 0
    # no keys: accumulators unchanged, nothing enqueued
    assert _decode(lib, _dims(q_len=1, kv_len=0), kv=None, op=None, lp=None) == 0


def _decode_noalloc(lib, dims, kc=64, q=FAKE, kv=FAKE2, o=ctypes.c_void_p(0x10000000),
                    lse=ctypes.c_void_p(0x20000000)):
    return lib.ring_attn_fwd_decode_noalloc(q, kv, kc, o, lse,
                                            ctypes.byref(dims) if dims is not None else None,
                                            None)


def test_decode_noalloc_limit_and_validation(lib):
    """The allocation-free decode step validates like ring_attn_fwd_decode and
    rejects, before touching the device, splits whose partials exceed the
    library's scratch array."""
    text = open(HEADER).read()
    m = re.search(r"#define RA_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.DECODE_SCRATCH_BYTES
    d1 = _dims(q_len=1, kv_len=4096)
    assert _decode_noalloc(lib, None) == -1
    assert _decode_noalloc(lib, _dims(q_len=1, dtype=1)) == -2
    assert _decode_noalloc(lib, _dims(heads=2, q_len=65)) == -2
    assert _decode_noalloc(lib, d1, kc=0) == -1
    assert _decode_noalloc(lib, d1, q=None) == -1
    assert _decode_noalloc(lib, d1, o=ctypes.c_void_p(0x1000)) == -1   # o_acc aliases q
    # 64 x 64 rows, 512 splits of 128 keys: 1 GiB of partials > 16 MiB
    far = dict(q=ctypes.c_void_p(1 << 40), kv=ctypes.c_void_p(2 << 40),
               o=ctypes.c_void_p(3 << 40), lse=ctypes.c_void_p(4 << 40))
    big = _dims(batch=64, heads=64, q_len=1, kv_len=65536)
    assert _decode_noalloc(lib, big, kc=128, **far) == -1
    assert b"scratch" in lib.ring_attn_last_error()
    # one split past the limit: S * rows * (4 d + 4) bytes
    rows = 8 * 32                                   # B = 8, H = 32, Lq = 1
    s_max = _lib.DECODE_SCRATCH_BYTES // (rows * 129 * 4)
    over = _dims(batch=8, heads=32, q_len=1, kv_len=(s_max + 1) * 64)
    assert _decode_noalloc(lib, over, kc=64, **far) == -1
    assert b"scratch" in lib.ring_attn_last_error()
    nul = dict(q=None, kv=None, o=None, lse=None)
    assert _decode_noalloc(lib, _dims(q_len=0), **nul) == 0
    assert _decode_noalloc(lib, _dims(q_len=1, kv_len=0), kv=None) == 0


def test_decode_split_planning(lib):
    def chunk(**kw):
        return lib.ring_attn_decode_chunk(ctypes.byref(_dims(**kw)))

    def splits(kc, **kw):
        return lib.ring_attn_decode_splits(ctypes.byref(_dims(**kw)), kc)

    # about one workgroup per compute unit (B * Hkv * S ~ 256), at most 8192
    # keys per split, whole tiles of 128 keys, at least four tiles
    assert chunk(batch=1, heads=32, q_len=1, kv_len=16384) == 2048
    assert chunk(batch=1, heads=32, kv_heads=8, q_len=4, kv_len=16384) == 512
    assert chunk(batch=8, heads=32, q_len=1, kv_len=16384) == 8192
    assert chunk(batch=8, heads=32, kv_heads=8, q_len=1, kv_len=16384) == 4096
    assert chunk(batch=8, heads=32, q_len=1, kv_len=131072) == 8192
    assert chunk(batch=1, heads=32, q_len=1, kv_len=100) == 512        # at least four tiles
    assert chunk(batch=1, heads=1, q_len=1, kv_len=1000) == 512
    assert chunk(q_len=1, dtype=1) == -2
    assert chunk(heads=8, kv_heads=1, q_len=9) == -2
    assert splits(2048, heads=32, q_len=1, kv_len=16384) == 8
    assert splits(200, q_len=1, kv_len=1000) == 5
    assert splits(1000, q_len=1, kv_len=1000) == 1
    assert splits(64, q_len=1, kv_len=0) == 0
    assert splits(0, q_len=1, kv_len=10) == -1
    for kw in ({"batch": 2, "heads": 16, "kv_heads": 2, "q_len": 4, "kv_len": 777},
               {"batch": 3, "heads": 5, "q_len": 1, "kv_len": 99999}):
        kc = chunk(**kw)
        assert kc > 0 and kc % 128 == 0
        assert splits(kc, **kw) <= 65536


def _ffn(lib, rows=300, dm=256, dff=512, chunk=128, x=FAKE, w1=ctypes.c_void_p(0x1000000),
         w2=ctypes.c_void_p(0x2000000), hidden=ctypes.c_void_p(0x10000000),
         out=ctypes.c_void_p(0x20000000)):
    return lib.ring_ffn_fwd(x, w1, w2, hidden, out, rows, dm, dff, chunk, None)


def test_ffn_rejects_invalid_and_unsupported(lib):
    assert _ffn(lib, dm=200) == -2                     # multiples of 256 only
    assert _ffn(lib, dff=640) == -2
    assert _ffn(lib, dm=0) == -2
    assert _ffn(lib, rows=-1) == -1
    assert _ffn(lib, rows=1 << 31) == -1
    assert _ffn(lib, chunk=0) == -1
    assert _ffn(lib, x=None) == -1
    assert _ffn(lib, hidden=None) == -1
    assert _ffn(lib, out=None) == -1
    # x [300, 256] bf16 spans 150 KiB from 0x1000
    assert _ffn(lib, out=ctypes.c_void_p(0x1000 + 4096)) == -1          # out overlaps x
    assert _ffn(lib, hidden=ctypes.c_void_p(0x2000000 + 64)) == -1      # hidden overlaps w2
    assert _ffn(lib, hidden=ctypes.c_void_p(0x20000000 - 1024)) == -1   # hidden overlaps out
    assert b"multiples of 256" in (_ffn(lib, dm=96) and lib.ring_attn_last_error())


def test_ffn_empty_is_a_no_op(lib):
    assert _ffn(lib, rows=0, x=None, w1=None, w2=None, hidden=None, out=None) == 0


def test_ffn_bwd_workspace_size(lib):
    ws = lib.ring_ffn_bwd_workspace
    # W1^T, W2^T; Z, G [c x dff]; x^T, dout^T [dm x cp]; G^T, H^T [dff x cp]
    dm, dff, c = 256, 512, 300
    cp = 320
    want = 2 * (dm * dff * 2) + 2 * (c * dff * 2) + 2 * (dm * cp * 2) + 2 * (dff * cp * 2)
    assert ws(300, dm, dff, 4096) == want          # chunk larger than rows: c = rows
    assert ws(1000, dm, dff, 300) == want
    assert ws(0, dm, dff, 64) > 0
    assert ws(10, 200, dff, 64) == -2
    assert ws(10, dm, dff, 0) == -1
    assert ws(10, 1 << 22, 1 << 22, 64) == -1      # weight transposes beyond one grid


def _ffn_bwd(lib, rows=300, dm=256, dff=512, chunk=128, work_bytes=1 << 30, **ptrs):
    p = dict(x=FAKE, w1=ctypes.c_void_p(0x1000000), w2=ctypes.c_void_p(0x2000000),
             dout=ctypes.c_void_p(0x3000000), dx=ctypes.c_void_p(0x4000000),
             dw1=ctypes.c_void_p(0x5000000), dw2=ctypes.c_void_p(0x6000000),
             work=ctypes.c_void_p(0x10000000))
    p.update(ptrs)
    return lib.ring_ffn_bwd(p["x"], p["w1"], p["w2"], p["dout"], p["dx"], p["dw1"], p["dw2"],
                            p["work"], work_bytes, rows, dm, dff, chunk, None)


def test_ffn_bwd_rejects_invalid(lib):
    assert _ffn_bwd(lib, dm=128) == -2
    assert _ffn_bwd(lib, chunk=0) == -1
    assert _ffn_bwd(lib, rows=-3) == -1
    for name in ("x", "w1", "w2", "dout", "dx", "dw1", "dw2", "work"):
        assert _ffn_bwd(lib, **{name: None}) == -1, name
    assert _ffn_bwd(lib, work_bytes=1000) == -1                          # workspace too small
    assert b"workspace" in lib.ring_attn_last_error()
    assert _ffn_bwd(lib, dx=ctypes.c_void_p(0x1000 + 512)) == -1         # dx overlaps x
    assert _ffn_bwd(lib, dw2=ctypes.c_void_p(0x5000000 + 4096)) == -1    # dw2 overlaps dw1
    assert _ffn_bwd(lib, work=ctypes.c_void_p(0x3000000 + 64)) == -1     # work overlaps dout
    none = {k: None for k in ("x", "w1", "w2", "dout", "dx", "dw1", "dw2", "work")}
    assert _ffn_bwd(lib, rows=0, work_bytes=0, **none) == 0              # nothing to do


def test_timing_families_documented_in_the_header_are_accepted(lib):
    """Every kernel family the header lists can be read back (no records
    here: zero launches, no GPU call), and an unknown one is rejected."""
    text = open(HEADER).read()
    block = text[text.index("kernel timing (diagnostics)"):text.index("ring_attn_timing_enable(on)")]
    names = re.findall(r'"([a-z0-9_]+)"', block)
    assert {"fwd_bf16", "bwd_dkv", "fwd_decode", "ffn_up", "ffn_bwd_gemm"} <= set(names)
    n, ms = ctypes.c_int(-1), ctypes.c_double(-1.0)
    for name in names:
        assert lib.ring_attn_timing_read(name.encode(), ctypes.byref(n), ctypes.byref(ms)) == 0
        assert n.value == 0 and ms.value == 0.0
    assert lib.ring_attn_timing_read(b"no_such_family", ctypes.byref(n), ctypes.byref(ms)) == -1


def test_emulator_rejects_bad_schedules(lib):
    d = _dims()
    pool = (ctypes.c_void_p * 2)(FAKE2.value, 0x300000)
    bad_order = (ctypes.c_int32 * 2)(0, 0)
    rc = lib.ring_emu_fwd(FAKE, pool, None, None, 0, 2, 0, 64, 64,
                          ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x20000000),
                          ctypes.byref(d), bad_order, 0, None, None)
    assert rc == -1 and b"permutation" in lib.ring_attn_last_error()
    rc = lib.ring_emu_fwd(FAKE, pool, None, None, 0, 2, 0, 64, 64,
                          ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x20000000),
                          ctypes.byref(d), None, 5, None, None)
    assert rc == -1 and b"mode" in lib.ring_attn_last_error()
    # two blocks need a receive slot; none given (any valid mode, unsafe too)
    for mode in (0, 1, 2):
        rc = lib.ring_emu_fwd(FAKE, pool, None, None, 0, 2, 0, 64, 64,
                              ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x20000000),
                              ctypes.byref(d), None, mode, None, None)
        assert rc == -1 and b"slot" in lib.ring_attn_last_error()
    rc = lib.ring_emu_fwd(FAKE, pool, None, None, 0, 2, 0, 64, 64,
                          ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x20000000),
                          ctypes.byref(d), None, 3, None, None)
    assert rc == -1 and b"mode" in lib.ring_attn_last_error()


def test_emulator_modes_match_the_header():
    text = open(HEADER).read()
    m = re.search(r"enum \{ RA_EMU_OVERLAP = (\d), RA_EMU_SERIALIZE = (\d), RA_EMU_UNSAFE = (\d) \}", text)
    assert m and tuple(int(x) for x in m.groups()) == (
        _lib.RA_EMU_OVERLAP, _lib.RA_EMU_SERIALIZE, _lib.RA_EMU_UNSAFE)
    assert _lib._emu_mode(False, False) == _lib.RA_EMU_OVERLAP
    assert _lib._emu_mode(True, False) == _lib.RA_EMU_SERIALIZE
    assert _lib._emu_mode(False, True) == _lib.RA_EMU_UNSAFE
    with pytest.raises(ValueError):
        _lib._emu_mode(True, True)


def test_bench_trace_overlap_report(tmp_path, capsys):
    """The copy/compute overlap report of bench.py on a hand-made trace."""
    import json
    import bench
    path = tmp_path / "trace.csv"
    cols = ["Queue_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [("1", "void fwd_bf16_kernel<128, 64, 8>(...)", 100, 200),
            ("1", "void dq_kernel<128, 64, 8>(...)", 200, 300),
            ("2", "__amd_rocclr_copyBuffer", 150, 250),   # fully under attention
            ("2", "__amd_rocclr_copyBuffer", 280, 380)]   # 20 of 100 under attention
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(cols)
        w.writerows(rows)
    bench._trace_overlap(str(path))
    out = json.loads(capsys.readouterr().out)
    assert out["copy_kernels"] == 2
    assert out["overlap_fraction"] == round(120 / 200, 4)
    assert out["copy_queues"] == ["2"] and out["attention_queues"] == ["1"]


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one member's share on one GPU: --gpus 2 exits with a
    message and a non-zero status before touching any device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
