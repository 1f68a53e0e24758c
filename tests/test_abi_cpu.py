"""The C-ABI library on the CPU: it loads, exports every function that
include/pdllm.h declares, plans deterministically, and rejects bad
arguments with the documented status codes before touching a device.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = pytest.importorskip("diffusion_long_context_amd._lib")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


def _declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    return set(re.findall(r"\b(pdllm_[a-zA-Z_0-9]+)\s*\(", text))


def test_every_declared_symbol_is_exported():
    names = _declared("pdllm.h")
    assert len(names) >= 9
    for n in names:
        assert hasattr(L.lib, n), f"{n} declared in include/pdllm.h but not exported"
    assert set(L.EXPORTS) <= names
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == \
        ["pdllm.h", "pdllm_calib.h"]


def test_calibration_library_exports_its_header():
    """The peak-calibration library (measurement only) loads on the CPU and
    exports what include/pdllm_calib.h declares; the path library does not
    carry those symbols."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "diffusion_long_context_amd", "libpdllm_calib.so"))
    names = _declared("pdllm_calib.h")
    assert len(names) == 4
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/pdllm_calib.h but not exported"
        assert not hasattr(L.lib, n)
    lib.pdllm_calib_mfma_bf16_flops.restype = ctypes.c_int64
    lib.pdllm_calib_mfma_bf16_flops.argtypes = [ctypes.c_int64, ctypes.c_int32]
    assert lib.pdllm_calib_mfma_bf16_flops(3, 5) == 5 * 4 * 3 * 4 * 32 * 32 * 16 * 2


def test_abi_version():
    assert L.lib.pdllm_abi_version() == 11


def _pool(**kw):
    f = dict(k=0x10000, v=0x20000, stride_slot=257 * 4 * 128, stride_row=4 * 128, stride_head=128,
             n_slots=128, slot_rows=257, h_kv=4, d=128, dtype=1)
    f.update(kw)
    return L.Pool(f["k"], f["v"], f["stride_slot"], f["stride_row"], f["stride_head"], f["n_slots"],
                  f["slot_rows"], f["h_kv"], f["d"], f["dtype"])


def _pt(ks, **kw):
    arr = (ctypes.c_int32 * len(ks))(*ks)
    f = dict(chunk_slot=0x30000, sel_chunk=0x40000, keep_rows=0x50000, n_chunks_per_seq=128,
             k_max=16, b=256, rows_compacted=0)
    f.update(kw)
    pt = L.PageTable(f["chunk_slot"], f["sel_chunk"], f["keep_rows"], ctypes.cast(arr, ctypes.c_void_p),
                     f["n_chunks_per_seq"], f["k_max"], f["b"], f["rows_compacted"])
    return pt, arr


def _decode(pool, pt, n_seq=1, l_d=256, h_q=28, ws=None, ws_bytes=0, q=0x60000, o=0x90000, scale=0.088,
            splits=0):
    return L.lib.pdllm_split_attn_decode(ctypes.byref(pool) if pool is not None else None,
                                         ctypes.byref(pt) if pt is not None else None,
                                         q, 0x70000, 0x80000, n_seq, l_d, h_q, scale, splits, o, None,
                                         ws, ws_bytes, None)


def _err():
    return L.lib.pdllm_last_error().decode()


@pytest.mark.parametrize("mutate,code,msg", [
    (dict(pool=None), INVALID, "pool is NULL"),
    (dict(dtype=7), INVALID, "dtype"),
    (dict(d=96), UNSUPPORTED, "head dim"),
    (dict(h_q=27), INVALID, "multiple of h_kv"),
    (dict(l_d=0), INVALID, ">= 1"),
    (dict(k_per_seq=[17]), INVALID, "k_per_seq[0]"),
    (dict(k_per_seq=[-1]), INVALID, "k_per_seq[0]"),
    (dict(b=257), INVALID, "b 257"),
    (dict(k_max=129), INVALID, "k_max"),
    (dict(stride_head=64), INVALID, "strides"),
    (dict(stride_head=132), INVALID, "multiples"),
    (dict(k=0x10008), INVALID, "aligned"),
    (dict(q=0), INVALID, "q is NULL"),
    (dict(o=0x90004), INVALID, "aligned"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(scale=0.0), INVALID, "scale"),
    (dict(scale=-0.088), INVALID, "scale"),
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(splits=-1), INVALID, "num_splits"),
    (dict(keep_rows=None), INVALID, "keep_rows is NULL"),
    (dict(rows_compacted=2), INVALID, "rows_compacted"),
    (dict(keep_rows=None, rows_compacted=1), WS_SMALL, "workspace"),   # compacted: keep_rows unread
    (dict(), WS_SMALL, "workspace"),
])
def test_decode_validation(mutate, code, msg):
    pool_kw = {k: mutate[k] for k in ("dtype", "d", "stride_head", "stride_row", "k") if k in mutate}
    pool = None if "pool" in mutate else _pool(**pool_kw)
    pt_kw = {k: mutate[k] for k in ("b", "k_max", "keep_rows", "rows_compacted") if k in mutate}
    pt, _keep = _pt(mutate.get("k_per_seq", [16]), **pt_kw)
    call = {k: mutate[k] for k in ("h_q", "l_d", "q", "o", "scale", "splits") if k in mutate}
    st = _decode(pool, pt, **call)
    assert st == code, _err()
    assert msg in _err()


def test_decode_null_tables_when_no_chunk_is_selected():
    """With every K_s = 0 the index tables are not read, so NULL is accepted
    (validation passes and stops at the workspace check of a two-split plan);
    with any K_s > 0 NULL chunk_slot / sel_chunk is rejected."""
    pool = _pool()
    pt, _keep = _pt([0, 0], chunk_slot=None, sel_chunk=None, keep_rows=None)
    assert _decode(pool, pt, n_seq=2, splits=2) == WS_SMALL, _err()
    pt, _keep = _pt([0, 3], chunk_slot=None, sel_chunk=None, keep_rows=None)
    assert _decode(pool, pt, n_seq=2) == INVALID and "chunk_slot" in _err()


def _decode_ex(pool, pt, opts, ws=None, ws_bytes=0):
    return L.lib.pdllm_split_attn_decode_ex(ctypes.byref(pool), ctypes.byref(pt), 0x60000, 0x70000, 0x80000,
                                            1, 256, 28, 0.088, ctypes.byref(opts) if opts is not None else None,
                                            0x90000, None, ws, ws_bytes, None)


def test_decode_options_validation():
    pool = _pool()
    pt, _keep = _pt([16])
    assert _decode_ex(pool, pt, None) == INVALID and "options" in _err()
    assert _decode_ex(pool, pt, L.DecodeOpts(0, 96)) == UNSUPPORTED and "q_rows_per_wg" in _err()
    assert _decode_ex(pool, pt, L.DecodeOpts(0, 64)) == UNSUPPORTED          # the f32 kernel's shape
    bad = L.DecodeOpts(0, 0)
    bad.reserved[3] = 1
    assert _decode_ex(pool, pt, bad) == INVALID and "reserved" in _err()
    for rows in (0, 128, 256):
        opts = L.DecodeOpts(0, rows)
        need = L.lib.pdllm_split_attn_decode_ex_workspace(ctypes.byref(pool), ctypes.byref(pt), 1, 256, 28,
                                                          ctypes.byref(opts))
        assert need > 0
        assert _decode_ex(pool, pt, opts, 0x100000, need - 1) == WS_SMALL
    f32 = _pool(dtype=0)
    assert _decode_ex(f32, pt, L.DecodeOpts(0, 128)) == UNSUPPORTED
    assert _decode_ex(f32, pt, L.DecodeOpts(0, 64)) == WS_SMALL


def test_decode_forced_shape_plans():
    """q_rows_per_wg fixes the planner's workgroup shape; the plain call's
    workspace equals the options call's with the same split count."""
    pool = _pool()
    pt, _keep = _pt([16])
    q = lambda rows, ns, merge=0: L.lib.pdllm_split_attn_decode_ex_workspace(
        ctypes.byref(pool), ctypes.byref(pt), 1, 256, 28, ctypes.byref(L.DecodeOpts(ns, rows, merge)))
    for ns in (0, 3):
        assert q(0, ns) == L.lib.pdllm_split_attn_decode_workspace(ctypes.byref(pool), ctypes.byref(pt), 1, 256,
                                                                   28, ns)
    # forced split counts, separate merge kernel: bf16 partials + float32 lse,
    # independent of the workgroup shape
    part = 5 * 256 * 28 * 128 * 2
    lse = 5 * 256 * 28 * 4
    assert q(128, 5, 1) == q(256, 5, 1) == q(0, 5, 1) == part + lse
    # in-kernel merge: sync words first -- 2 + one arrival and rows / 32
    # claim words per (kv head, query tile) group -- then the partials (bf16
    # by default and with merge 3, float32 with merge 2) and float32 lse
    for rows in (128, 256):
        groups = 4 * (256 * 7 // rows)
        sync = -(-4 * (2 + groups * (1 + rows // 32)) // 256) * 256
        assert q(rows, 5, 3) == sync + part + lse
        assert q(rows, 5, 2) == sync + 2 * part + lse
        assert q(rows, 5) == part + lse                 # the default: a separate merge kernel
        assert q(rows, 5, 4) == 2 * part + lse          # separate merge kernel over float32 partials
    assert L.lib.pdllm_split_attn_decode_ex_workspace(ctypes.byref(_pool(dtype=0)), ctypes.byref(pt), 1, 256, 28,
                                                      ctypes.byref(L.DecodeOpts(5, 0, 2))) == 0
    assert "bf16 only" in _err()
    # float32 inputs keep float32 partials: merge 4 is merge 1
    f32q = lambda merge: L.lib.pdllm_split_attn_decode_ex_workspace(
        ctypes.byref(_pool(dtype=0)), ctypes.byref(pt), 1, 256, 28, ctypes.byref(L.DecodeOpts(5, 64, merge)))
    assert f32q(4) == f32q(1) == 2 * part + lse
    assert q(0, 5, 5) == 0 and "merge" in _err()


def test_noalloc_decode_validation():
    """The no-allocation decode validates like the workspace call and
    rejects, before touching a device, a plan whose partials exceed its
    64 MiB scratch."""
    f = L.lib.pdllm_split_attn_decode_noalloc
    pool = _pool()
    pt, _keep = _pt([16])
    call = lambda **kw: f(ctypes.byref(pool), ctypes.byref(kw.get("pt", pt)), kw.get("q", 0x60000), 0x70000,
                          0x80000, 1, 256, kw.get("h_q", 28), kw.get("scale", 0.088), kw.get("splits", 0),
                          0x90000, None, None)
    assert call(h_q=27) == INVALID and "multiple" in _err()
    assert call(q=0) == INVALID and "q is NULL" in _err()
    assert call(scale=0.0) == INVALID and "scale" in _err()
    # 69 splits x 256 rows x 28 heads x 128 d of bf16 partials: about 127 MB
    assert call(splits=69) == UNSUPPORTED and "scratch" in _err()


def test_decode_workspace_query_matches_plan():
    pool = _pool()
    pt, _keep = _pt([16])
    ws = L.lib.pdllm_split_attn_decode_workspace(ctypes.byref(pool), ctypes.byref(pt), 1, 256, 28, 0)
    splits, tps, plan_ws = L.decode_plan([16], 256, 256, 28, 4, 128, 1, 0, n_cu=256)
    assert ws == plan_ws > 0
    assert splits[0] > 1


def test_prefill_validation():
    pool = _pool()
    f = L.lib.pdllm_chunk_prefill_score
    args = lambda **kw: [ctypes.byref(kw.get("pool", pool)), 0x30000, None, kw.get("n", 128), 0x60000,
                         kw.get("h_q", 28), 0x70000, kw.get("w", 64), kw.get("cpw", 128), 0.088, 0x90000,
                         0xA0000, kw.get("ws", None), kw.get("ws_bytes", 0), None]
    assert f(*args(h_q=30)) == INVALID
    assert f(*args(w=0)) == INVALID
    assert f(*args(cpw=0)) == INVALID
    assert f(*args()) == WS_SMALL
    ws = L.lib.pdllm_prefill_score_workspace
    need = ws(128, 28, 4, 257, 64)
    assert need >= 128 * 4 * 8 * 257 * 4                      # per-wave partial rows
    # streamed chunks: one partial row per (chunk, kv head) + the window normalisers
    need_s = ws(8, 28, 4, 4097, 64)
    assert need_s >= 8 * 4 * 4097 * 4 + 8 * 4 * 448 * 4
    assert ws(8, 28, 4, 4097, 0) == 0 and ws(8, 30, 4, 4097, 64) == 0
    assert f(*args(pool=_pool(slot_rows=1025, stride_slot=1025 * 512), ws=0x100000,
                   ws_bytes=ws(128, 28, 4, 1025, 64) - 1)) == WS_SMALL
    assert f(*args(pool=_pool(slot_rows=4098, stride_slot=4098 * 512))) == UNSUPPORTED
    assert f(*args(n=0)) == OK                       # nothing to do, nothing enqueued
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        a = args()
        a[9] = bad
        assert f(*a) == INVALID and "scale" in _err()


def test_select_validation():
    tb = L.lib.pdllm_select_topB
    assert tb(0x1000, None, 4, 33, 33, 0x2000, None) == INVALID          # b > slot_rows - 1
    assert tb(0x1000, None, 4, 5000, 3, 0x2000, None) == UNSUPPORTED
    assert tb(0x1000, None, -1, 33, 3, 0x2000, None) == INVALID
    assert tb(0x1000, None, 4, 33, 0, 0x2000, None) == OK                # b = 0: nothing to do
    tk = L.lib.pdllm_select_topK
    ks = (ctypes.c_int32 * 2)(3, 9)
    assert tk(0x1000, 2, 8, ks, 8, 0x2000, None) == INVALID        # K_s > k_max
    assert tk(0x1000, 2, 8, ks, 9, 0x2000, None) == INVALID        # k_max > n_chunks
    assert tk(0x1000, 2, 9000, ks, 9, 0x2000, None) == UNSUPPORTED
    assert tk(0x1000, 0, 8, ks, 8, 0x2000, None) == OK


@pytest.mark.parametrize("ks,b,l_d,g,dtype", [
    ([16], 256, 256, 7, 1), ([8], 128, 256, 7, 1), ([8, 16, 24, 32], 128, 512, 7, 1),
    ([2], 16, 32, 1, 0), ([0, 1, 40], 7, 3, 2, 1), ([5], 0, 1, 1, 0),
])
def test_plan_properties(ks, b, l_d, g, dtype):
    h_kv = 4 if g == 7 else 2
    h_q = g * h_kv
    d = 128 if dtype else 64
    for num_splits in (0, 1, 2, 3, 1000):
        a = L.decode_plan(ks, b, l_d, h_q, h_kv, d, dtype, num_splits)
        assert a == L.decode_plan(ks, b, l_d, h_q, h_kv, d, dtype, num_splits)   # deterministic
        splits, tps, ws = a
        need = 0
        for s, k in enumerate(ks):
            n_tiles = -(-(k * (b + 1) + l_d) // 64)
            assert splits[s] >= 1 and tps[s] >= 1
            assert (splits[s] - 1) * tps[s] < n_tiles <= splits[s] * tps[s]
            if num_splits:
                assert splits[s] <= min(num_splits, n_tiles)
            if splits[s] > 1:   # partial O (bf16 for bf16 inputs, else float32) + float32 lse
                need += splits[s] * l_d * h_q * (d * (2 if dtype else 4) + 4)
        assert (ws == 0) == (need == 0) and ws >= need


def test_plan_rejects_bad_sizes():
    with pytest.raises(L.PdllmError):
        L.decode_plan([4], 8, 16, 6, 4, 128, 1)
    with pytest.raises(L.PdllmError):
        L.decode_plan([-1], 8, 16, 8, 4, 128, 1)


def test_chunk_score_validation():
    f = L.lib.pdllm_chunk_score
    ws = L.lib.pdllm_chunk_score_workspace
    assert ws(128, 64, 64) == 128 * 128 * 4
    assert ws(-1, 64, 64) == 0
    need = ws(4, 3, 5)
    args = lambda **kw: [kw.get("logits", 0x100000), kw.get("dtype", 1), kw.get("stride", 152064),
                         kw.get("vocab", 152064), 0x200000, kw.get("n", 4), kw.get("nq", 3), kw.get("np_", 5),
                         None, None, kw.get("s", 0x300000), kw.get("ws", 0x400000), kw.get("ws_bytes", need), None]
    assert f(*args(dtype=7)) == INVALID
    assert f(*args(vocab=0)) == INVALID
    assert f(*args(stride=100, vocab=101)) == INVALID
    assert f(*args(stride=152065)) == INVALID                     # rows not 16-byte aligned
    assert f(*args(logits=0x100002)) == INVALID                   # base not 16-byte aligned
    assert f(*args(s=None)) == INVALID
    assert f(*args(nq=-1)) == INVALID
    assert f(*args(ws_bytes=need - 1)) == WS_SMALL
    assert f(*args(n=0)) == OK                                      # nothing to do, nothing enqueued


def test_compaction_validation():
    f = L.lib.pdllm_compact_kept_rows
    pool = _pool()
    # destination: [128][b + 1 = 129][4][128] dense
    args = lambda **kw: [ctypes.byref(kw.get("pool", pool)), kw.get("slot", 0x30000), kw.get("n", 128),
                         kw.get("keep", 0x50000), kw.get("b", 128), kw.get("dk", 0x100000), kw.get("dv", 0x200000),
                         kw.get("ss", 129 * 512), kw.get("sr", 512), kw.get("sh", 128), kw.get("rows", 129), None]
    assert f(*args(b=257)) == INVALID                      # b > slot_rows - 1
    assert "b 257" in _err()
    assert f(*args(b=-1)) == INVALID
    assert f(*args(rows=128)) == INVALID                   # dst_slot_rows < b + 1
    assert "dst_slot_rows" in _err()
    assert f(*args(ss=128 * 512)) == INVALID               # dst slots overlap
    assert f(*args(sh=132)) == INVALID                     # dst stride not a multiple of 8
    assert f(*args(dk=0x100008)) == INVALID                # dst not 16-byte aligned
    assert f(*args(dv=None)) == INVALID
    assert f(*args(keep=None)) == INVALID
    assert "keep_rows is NULL" in _err()
    assert f(*args(slot=None)) == INVALID
    assert f(*args(n=-1)) == INVALID
    assert f(*args(pool=_pool(d=96))) == UNSUPPORTED
    assert f(*args(n=0)) == OK                              # nothing to do, nothing enqueued


def test_prefill_select_validation():
    f = L.lib.pdllm_prefill_select
    pool = _pool()
    ks = (ctypes.c_int32 * 2)(16, 16)
    ws = L.lib.pdllm_prefill_score_workspace(128, 28, 4, 257, 64)
    args = lambda **kw: [ctypes.byref(kw.get("pool", pool)), 0x30000, None, kw.get("n", 128), 0x60000, 28,
                         0x70000, 64, 128, 0.088, 0x90000, 0xA0000, kw.get("b", 256), kw.get("keep", 0xB0000),
                         kw.get("cs", 0xC0000), kw.get("n_seq", 1), kw.get("ks", ks), kw.get("k_max", 16),
                         kw.get("sel", 0xD0000), kw.get("so", 0), kw.get("ws", 0x100000), kw.get("ws_bytes", ws),
                         None]
    assert f(*args(b=257)) == INVALID and "b 257" in _err()
    assert f(*args(keep=None)) == INVALID and "keep_rows" in _err()
    assert f(*args(n_seq=3)) == INVALID and "divide" in _err()
    assert f(*args(k_max=129)) == INVALID and "k_max" in _err()
    assert f(*args(ks=(ctypes.c_int32 * 1)(17))) == INVALID and "k_per_seq[0]" in _err()
    assert f(*args(cs=None)) == INVALID
    assert f(*args(sel=None)) == INVALID
    assert f(*args(ws_bytes=ws - 1)) == WS_SMALL
    assert f(*args(pool=_pool(d=96))) == UNSUPPORTED
    assert f(*args(so=2)) == INVALID and "selected_only" in _err()
    assert f(*args(so=1, cs=None, k_max=0)) == INVALID and "chunk_score" in _err()
    assert f(*args(n=0, n_seq=1, k_max=0)) == OK        # nothing to do, nothing enqueued


def test_decode_no_split_shape_validation():
    """q_rows_per_wg = 32 (the decode without kv splits) needs no workspace,
    takes bf16 only, no split count above 1, no merge option other than the
    default, and at most 4864 pool rows per sequence."""
    pool = _pool()
    pt, _keep = _pt([16])
    ws = lambda opts, p=pool, t=pt: L.lib.pdllm_split_attn_decode_ex_workspace(
        ctypes.byref(p), ctypes.byref(t), 1, 256, 28, ctypes.byref(opts))
    assert ws(L.DecodeOpts(0, 32)) == 0 and ws(L.DecodeOpts(1, 32)) == 0
    assert ws(L.DecodeOpts(2, 32)) == 0 and "32-row" in _err()
    assert ws(L.DecodeOpts(0, 32, 4)) == 0 and "32-row" in _err()
    assert _decode_ex(_pool(dtype=0), pt, L.DecodeOpts(0, 32)) == UNSUPPORTED
    big, _keep2 = _pt([20], b=255, k_max=20)              # 20 x 256 pool rows > 4864
    assert ws(L.DecodeOpts(0, 32), t=big) == 0 and "4864" in _err()
    # a plan with no workspace validates up to the launch; this one stops at
    # the NULL output check
    assert L.lib.pdllm_split_attn_decode_ex(ctypes.byref(pool), ctypes.byref(pt), 0x60000, 0x70000, 0x80000, 1,
                                            256, 28, 0.088, ctypes.byref(L.DecodeOpts(0, 32)), None, None, None,
                                            0, None) == INVALID


def test_planner_takes_the_no_split_decode_where_it_measured_faster():
    """The planner's choice between the split decode and the decode without
    splits (q_rows_per_wg = 32) on the workloads it was measured on: the 8K
    workload (1,288 attended rows) takes no splits; the 32K and full-step
    layers, the 128K batch and small windows (few query rows) keep splits;
    f32 and a forced split count never take it."""
    import synth
    for name, rows in (("s8", 32), ("s32", 256), ("f32", 256), ("s128", 256)):
        c = synth.config(name)
        splits, tps, ws, got = L.decode_plan(c.k_per_seq, c.b, c.l_d, c.h_q, c.h_kv, c.d, 1, with_rows=True)
        assert got == rows, f"{name}: planner chose {got}-row workgroups"
        if rows == 32:
            assert ws == 0 and splits == [1] * len(c.k_per_seq)
    for l_d in (16, 32):
        c = synth.config("s32", l_d=l_d)
        assert L.decode_plan(c.k_per_seq, c.b, c.l_d, c.h_q, c.h_kv, c.d, 1, with_rows=True)[3] == 256
    c = synth.config("s8")
    assert L.decode_plan(c.k_per_seq, c.b, c.l_d, c.h_q, c.h_kv, c.d, 1, num_splits=3, with_rows=True)[3] == 256
    assert L.decode_plan(c.k_per_seq, c.b, c.l_d, c.h_q, c.h_kv, c.d, 0, with_rows=True)[3] == 64


def test_resolve_rows_validation():
    """pdllm_resolve_rows checks the pool, the page table and the output
    before anything is enqueued; a decode given resolved rows accepts NULL
    index tables and rejects a misaligned rows pointer."""
    f = L.lib.pdllm_resolve_rows
    pool = _pool()
    pt, _keep = _pt([16])
    need = 1 * 16 * 257
    assert f(ctypes.byref(pool), ctypes.byref(pt), 1, None, need, None) == INVALID and "rows is NULL" in _err()
    assert f(ctypes.byref(pool), ctypes.byref(pt), 1, 0xA0000, need - 1, None) == INVALID and "needed" in _err()
    assert f(ctypes.byref(pool), ctypes.byref(pt), 0, 0xA0000, need, None) == INVALID
    assert f(ctypes.byref(pool), None, 1, 0xA0000, need, None) == INVALID
    bad, _k = _pt([16], sel_chunk=None)
    assert f(ctypes.byref(pool), ctypes.byref(bad), 1, 0xA0000, need, None) == INVALID and "sel_chunk" in _err()
    assert f(ctypes.byref(_pool(dtype=0)), ctypes.byref(pt), 1, 0xA0000, need, None) == UNSUPPORTED
    huge = _pool(n_slots=1 << 20, stride_slot=1 << 20)
    assert f(ctypes.byref(huge), ctypes.byref(pt), 1, 0xA0000, need, None) == UNSUPPORTED
    # a decode over resolved rows: NULL tables accepted (validation runs to the workspace check)
    rpt, _k2 = _pt([16], chunk_slot=None, sel_chunk=None, keep_rows=None)
    rpt.rows = 0xA0000
    assert _decode(pool, rpt, splits=2) == WS_SMALL, _err()
    rpt.rows = 0xA0002
    assert _decode(pool, rpt, splits=2) == INVALID and "aligned" in _err()
    rpt.rows = 0xA0000
    assert _decode(_pool(dtype=0), rpt, splits=2) == UNSUPPORTED and "bf16" in _err()
