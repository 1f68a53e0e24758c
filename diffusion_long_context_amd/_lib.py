"""ctypes binding of libpdllm (include/pdllm.h) for torch tensors.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch provides device memory (outputs and workspaces are allocated
with ``torch.empty``) and the stream (the current HIP stream).  If the
library has not been built, importing this module raises ``ImportError``:
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpdllm.so")

F32, BF16 = 0, 1
_DTYPE = {torch.float32: F32, torch.bfloat16: BF16}


class Pool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("stride_slot", ctypes.c_int64), ("stride_row", ctypes.c_int64),
                ("stride_head", ctypes.c_int64), ("n_slots", ctypes.c_int32),
                ("slot_rows", ctypes.c_int32), ("h_kv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PageTable(ctypes.Structure):
    _fields_ = [("chunk_slot", ctypes.c_void_p), ("sel_chunk", ctypes.c_void_p),
                ("keep_rows", ctypes.c_void_p), ("k_per_seq", ctypes.c_void_p),
                ("n_chunks_per_seq", ctypes.c_int32), ("k_max", ctypes.c_int32),
                ("b", ctypes.c_int32), ("rows_compacted", ctypes.c_int32), ("rows", ctypes.c_void_p)]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("q_rows_per_wg", ctypes.c_int32),
                ("merge", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


EXPORTS = ("pdllm_prefill_score_workspace", "pdllm_chunk_prefill_score", "pdllm_select_topB",
           "pdllm_select_topK", "pdllm_decode_plan", "pdllm_split_attn_decode_workspace",
           "pdllm_split_attn_decode", "pdllm_last_error", "pdllm_abi_version",
           "pdllm_chunk_score_workspace", "pdllm_chunk_score", "pdllm_compact_kept_rows",
           "pdllm_prefill_select", "pdllm_split_attn_decode_ex_workspace", "pdllm_split_attn_decode_ex",
           "pdllm_split_attn_decode_noalloc", "pdllm_gather_kept_kv", "pdllm_resolve_rows")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m diffusion_long_context_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    P = ctypes.POINTER
    lib.pdllm_abi_version.restype = ctypes.c_int
    lib.pdllm_last_error.restype = ctypes.c_char_p
    lib.pdllm_prefill_score_workspace.restype = sz
    lib.pdllm_prefill_score_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.pdllm_chunk_prefill_score.restype = ctypes.c_int
    lib.pdllm_chunk_prefill_score.argtypes = [P(Pool), vp, vp, i32, vp, i32, vp, i32, i32, f32, vp, vp,
                                              vp, sz, vp]
    lib.pdllm_select_topB.restype = ctypes.c_int
    lib.pdllm_select_topB.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.pdllm_select_topK.restype = ctypes.c_int
    lib.pdllm_select_topK.argtypes = [vp, i32, i32, vp, i32, vp, vp]
    lib.pdllm_decode_plan.restype = ctypes.c_int
    lib.pdllm_decode_plan.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp,
                                      P(i32), P(i64)]
    lib.pdllm_split_attn_decode_workspace.restype = sz
    lib.pdllm_split_attn_decode_workspace.argtypes = [P(Pool), P(PageTable), i32, i32, i32, i32]
    lib.pdllm_split_attn_decode.restype = ctypes.c_int
    lib.pdllm_split_attn_decode.argtypes = [P(Pool), P(PageTable), vp, vp, vp, i32, i32, i32, f32,
                                            i32, vp, vp, vp, sz, vp]
    lib.pdllm_resolve_rows.restype = ctypes.c_int
    lib.pdllm_resolve_rows.argtypes = [P(Pool), P(PageTable), i32, vp, sz, vp]
    lib.pdllm_split_attn_decode_ex_workspace.restype = sz
    lib.pdllm_split_attn_decode_ex_workspace.argtypes = [P(Pool), P(PageTable), i32, i32, i32, P(DecodeOpts)]
    lib.pdllm_split_attn_decode_ex.restype = ctypes.c_int
    lib.pdllm_split_attn_decode_ex.argtypes = [P(Pool), P(PageTable), vp, vp, vp, i32, i32, i32, f32,
                                               P(DecodeOpts), vp, vp, vp, sz, vp]
    lib.pdllm_split_attn_decode_noalloc.restype = ctypes.c_int
    lib.pdllm_split_attn_decode_noalloc.argtypes = [P(Pool), P(PageTable), vp, vp, vp, i32, i32, i32, f32, i32,
                                                    vp, vp, vp]
    lib.pdllm_gather_kept_kv.restype = ctypes.c_int
    lib.pdllm_gather_kept_kv.argtypes = [P(Pool), P(PageTable), i32, vp, vp, i64, i64, i64, vp]
    lib.pdllm_chunk_score_workspace.restype = sz
    lib.pdllm_chunk_score_workspace.argtypes = [i32, i32, i32]
    lib.pdllm_chunk_score.restype = ctypes.c_int
    lib.pdllm_chunk_score.argtypes = [vp, i32, i64, i32, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.pdllm_prefill_select.restype = ctypes.c_int
    lib.pdllm_prefill_select.argtypes = [P(Pool), vp, vp, i32, vp, i32, vp, i32, i32, f32, vp, vp, i32, vp, vp,
                                         i32, vp, i32, vp, i32, vp, sz, vp]
    lib.pdllm_compact_kept_rows.restype = ctypes.c_int
    lib.pdllm_compact_kept_rows.argtypes = [P(Pool), vp, i32, vp, i32, vp, vp, i64, i64, i64, i32, vp]
    return lib


lib = _load()
ABI_VERSION = 11
if lib.pdllm_abi_version() != ABI_VERSION:
    raise ImportError(f"libpdllm ABI {lib.pdllm_abi_version()} != binding ABI {ABI_VERSION}")


class PdllmError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib.pdllm_last_error().decode(errors="replace")
        super().__init__(f"{what} failed with status {status}: {msg}")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != 0:
        raise PdllmError(status, what)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dense(t: torch.Tensor, name: str, dtype=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def make_pool(pool_k: torch.Tensor, pool_v: torch.Tensor) -> Pool:
    """Describe [n_slots][slot_rows][h_kv][d] K/V tensors (any strides with d
    contiguous; K and V must share strides)."""
    if pool_k.shape != pool_v.shape or pool_k.stride() != pool_v.stride():
        raise ValueError("pool k and v must have the same shape and strides")
    if pool_k.dtype not in _DTYPE or pool_v.dtype != pool_k.dtype:
        raise ValueError("pool dtype must be float32 or bfloat16 (both the same)")
    if pool_k.dim() != 4 or pool_k.stride(3) != 1:
        raise ValueError("pool tensors must be 4-D with the head dim contiguous")
    n_slots, rows, h_kv, d = pool_k.shape
    return Pool(pool_k.data_ptr(), pool_v.data_ptr(), pool_k.stride(0), pool_k.stride(1),
                pool_k.stride(2), n_slots, rows, h_kv, d, _DTYPE[pool_k.dtype])


def chunk_prefill_score(pool_k, pool_v, chunk_slot, q_chunk, q_win, chunks_per_win, scale,
                        o_chunk=None, key_score=None, workspace=None,
                        chunk_rows=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """pdllm_chunk_prefill_score.  q_chunk [n_chunks][R][h_q][d], q_win
    [n_win][W][h_q][d], chunk_rows [n_chunks] int32 or None (every chunk
    whole); returns (o_chunk, key_score [n_chunks][R] float32)."""
    pool = make_pool(pool_k, pool_v)
    _dense(chunk_slot, "chunk_slot", torch.int32)
    if chunk_rows is not None:
        _dense(chunk_rows, "chunk_rows", torch.int32)
        if chunk_rows.numel() < q_chunk.shape[0]:
            raise ValueError("chunk_rows must hold n_chunks entries")
    _dense(q_chunk, "q_chunk", pool_k.dtype)
    _dense(q_win, "q_win", pool_k.dtype)
    n_chunks, rows, h_q, d = q_chunk.shape
    if rows != pool.slot_rows or d != pool.d or q_win.shape[2:] != (h_q, d):
        raise ValueError("q_chunk / q_win shapes do not match the pool")
    w = q_win.shape[1]
    if chunks_per_win < 1 or q_win.shape[0] * chunks_per_win < n_chunks:
        raise ValueError("q_win must hold ceil(n_chunks / chunks_per_win) windows")
    if chunk_slot.numel() < n_chunks:
        raise ValueError("chunk_slot must hold n_chunks entries")
    dev = q_chunk.device
    if o_chunk is None:
        o_chunk = torch.empty_like(q_chunk)
    if key_score is None:
        key_score = torch.empty((n_chunks, rows), dtype=torch.float32, device=dev)
    need = lib.pdllm_prefill_score_workspace(n_chunks, h_q, pool.h_kv, rows, w)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib.pdllm_chunk_prefill_score(ctypes.byref(pool), chunk_slot.data_ptr(), _ptr(chunk_rows), n_chunks,
                                         q_chunk.data_ptr(), h_q, q_win.data_ptr(), w, chunks_per_win,
                                         float(scale), o_chunk.data_ptr(), key_score.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(), _stream(dev)),
           "pdllm_chunk_prefill_score")
    return o_chunk, key_score


def prefill_select(pool_k, pool_v, chunk_slot, q_chunk, q_win, chunks_per_win, scale, b, chunk_score,
                   k_per_seq: Sequence[int], k_max: int, chunk_rows=None, o_chunk=None, key_score=None,
                   keep_rows=None, sel_chunk=None, workspace=None, selected_only=False):
    """pdllm_prefill_select: chunk_prefill_score, select_topb and select_topk in
    one call (chunk_score [n_seq][n_chunks / n_seq] float32).  With
    selected_only, key_score and keep_rows are written for the chunks top-K
    selects only.  Returns (o_chunk, key_score, keep_rows, sel_chunk)."""
    pool = make_pool(pool_k, pool_v)
    _dense(chunk_slot, "chunk_slot", torch.int32)
    _dense(q_chunk, "q_chunk", pool_k.dtype)
    _dense(q_win, "q_win", pool_k.dtype)
    _dense(chunk_score, "chunk_score", torch.float32)
    n_chunks, rows, h_q, d = q_chunk.shape
    if rows != pool.slot_rows or d != pool.d or q_win.shape[2:] != (h_q, d):
        raise ValueError("q_chunk / q_win shapes do not match the pool")
    if chunks_per_win < 1 or q_win.shape[0] * chunks_per_win < n_chunks or chunk_slot.numel() < n_chunks:
        raise ValueError("q_win / chunk_slot do not cover n_chunks")
    if chunk_rows is not None:
        _dense(chunk_rows, "chunk_rows", torch.int32)
        if chunk_rows.numel() < n_chunks:
            raise ValueError("chunk_rows must hold n_chunks entries")
    n_seq = chunk_score.shape[0]
    if chunk_score.dim() != 2 or n_seq * chunk_score.shape[1] != n_chunks or len(k_per_seq) != n_seq:
        raise ValueError("chunk_score must be [n_seq][n_chunks / n_seq] with one K_s per sequence")
    dev = q_chunk.device
    o_chunk = torch.empty_like(q_chunk) if o_chunk is None else o_chunk
    if key_score is None:
        key_score = torch.empty((n_chunks, rows), dtype=torch.float32, device=dev)
    if keep_rows is None:
        keep_rows = torch.empty((n_chunks, b), dtype=torch.int32, device=dev)
    if sel_chunk is None:
        sel_chunk = torch.empty((n_seq, k_max), dtype=torch.int32, device=dev)
    need = lib.pdllm_prefill_score_workspace(n_chunks, h_q, pool.h_kv, rows, q_win.shape[1])
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    ks = (ctypes.c_int32 * max(n_seq, 1))(*[int(x) for x in k_per_seq])
    _check(lib.pdllm_prefill_select(ctypes.byref(pool), chunk_slot.data_ptr(), _ptr(chunk_rows), n_chunks,
                                    q_chunk.data_ptr(), h_q, q_win.data_ptr(), q_win.shape[1], chunks_per_win,
                                    float(scale), o_chunk.data_ptr(), key_score.data_ptr(), b, keep_rows.data_ptr(),
                                    chunk_score.data_ptr(), n_seq, ks, k_max, sel_chunk.data_ptr(),
                                    1 if selected_only else 0, workspace.data_ptr(), workspace.numel(), _stream(dev)),
           "pdllm_prefill_select")
    return o_chunk, key_score, keep_rows, sel_chunk


def select_topb(key_score: torch.Tensor, b: int, keep_rows=None, chunk_rows=None) -> torch.Tensor:
    """pdllm_select_topB: key_score [n_chunks][R] float32 -> [n_chunks][b] int32
    (-1 entries for a partial chunk of fewer than b content rows, given by
    chunk_rows [n_chunks] int32)."""
    _dense(key_score, "key_score", torch.float32)
    n_chunks, rows = key_score.shape
    if chunk_rows is not None:
        _dense(chunk_rows, "chunk_rows", torch.int32)
        if chunk_rows.numel() < n_chunks:
            raise ValueError("chunk_rows must hold n_chunks entries")
    if keep_rows is None:
        keep_rows = torch.empty((n_chunks, b), dtype=torch.int32, device=key_score.device)
    _check(lib.pdllm_select_topB(key_score.data_ptr(), _ptr(chunk_rows), n_chunks, rows, b, keep_rows.data_ptr(),
                                 _stream(key_score.device)), "pdllm_select_topB")
    return keep_rows


def select_topk(chunk_score: torch.Tensor, k_per_seq: Sequence[int], k_max: int,
                sel_chunk=None) -> torch.Tensor:
    """pdllm_select_topK: chunk_score [n_seq][N] float32 -> [n_seq][k_max] int32."""
    _dense(chunk_score, "chunk_score", torch.float32)
    n_seq, n = chunk_score.shape
    ks = (ctypes.c_int32 * max(n_seq, 1))(*[int(x) for x in k_per_seq])
    if sel_chunk is None:
        sel_chunk = torch.empty((n_seq, k_max), dtype=torch.int32, device=chunk_score.device)
    _check(lib.pdllm_select_topK(chunk_score.data_ptr(), n_seq, n, ks, k_max, sel_chunk.data_ptr(),
                                 _stream(chunk_score.device)), "pdllm_select_topK")
    return sel_chunk


def chunk_score(logits: torch.Tensor, target: torch.Tensor, n_query: int, n_pseudo: int,
                out=None, workspace=None):
    """pdllm_chunk_score: logits [n_chunks][n_query + n_pseudo][vocab] (bf16 or
    float32; the last dimension may be padded, rows 16-byte aligned), target
    [n_chunks][n_query + n_pseudo] int32 -> (s_i, s_p, s), each [n_chunks]
    float32."""
    if logits.dim() != 3 or (logits.numel() > 0 and (
            logits.stride(2) != 1 or logits.stride(0) != logits.shape[1] * logits.stride(1))):
        raise ValueError("logits must be [n_chunks][rows][vocab] with rows evenly spaced")
    if not logits.is_cuda:
        raise ValueError("logits must be a GPU tensor")
    dtype = {torch.float32: 0, torch.bfloat16: 1}.get(logits.dtype)
    if dtype is None:
        raise ValueError("logits must be float32 or bfloat16")
    _dense(target, "target", torch.int32)
    n_chunks, rows, vocab = logits.shape
    if rows != n_query + n_pseudo or target.shape != (n_chunks, rows):
        raise ValueError("logits / target shapes do not match n_query + n_pseudo")
    dev = logits.device
    if out is None:
        out = tuple(torch.empty(n_chunks, dtype=torch.float32, device=dev) for _ in range(3))
    need = lib.pdllm_chunk_score_workspace(n_chunks, n_query, n_pseudo)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib.pdllm_chunk_score(logits.data_ptr(), dtype, logits.stride(1), vocab, target.data_ptr(),
                                 n_chunks, n_query, n_pseudo, _ptr(out[0]), _ptr(out[1]), out[2].data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), _stream(dev)), "pdllm_chunk_score")
    return out


def compact_kept_rows(pool_k, pool_v, chunk_slot, keep_rows, dst_k=None, dst_v=None):
    """pdllm_compact_kept_rows: for chunk c in slot s = chunk_slot[c], writes
    the BOS row and the kept rows keep_rows[c] ([n_chunks][b] int32) to rows
    0..b of slot s of (dst_k, dst_v).  The destination defaults to new
    [n_slots][b + 1][h_kv][d] tensors (slots of no listed chunk are left
    uninitialised); returns (dst_k, dst_v)."""
    pool = make_pool(pool_k, pool_v)
    _dense(chunk_slot, "chunk_slot", torch.int32)
    _dense(keep_rows, "keep_rows", torch.int32)
    if keep_rows.dim() != 2:
        raise ValueError("keep_rows must be [n_chunks][b]")
    n_chunks, b = keep_rows.shape
    if chunk_slot.numel() < n_chunks:
        raise ValueError("chunk_slot must hold n_chunks entries")
    if dst_k is None:
        shape = (pool.n_slots, b + 1, pool.h_kv, pool.d)
        dst_k = torch.empty(shape, dtype=pool_k.dtype, device=pool_k.device)
        dst_v = torch.empty(shape, dtype=pool_k.dtype, device=pool_k.device)
    if dst_k.shape != dst_v.shape or dst_k.stride() != dst_v.stride() or dst_k.dtype != pool_k.dtype:
        raise ValueError("dst k and v must share shape, strides and the pool dtype")
    if dst_k.dim() != 4 or dst_k.stride(3) != 1 or dst_k.shape[0] != pool.n_slots or \
            dst_k.shape[2:] != (pool.h_kv, pool.d):
        raise ValueError("dst tensors must be [n_slots][rows][h_kv][d] with d contiguous")
    _check(lib.pdllm_compact_kept_rows(ctypes.byref(pool), chunk_slot.data_ptr(), n_chunks,
                                       _ptr(keep_rows) if b > 0 else None, b, dst_k.data_ptr(),
                                       dst_v.data_ptr(), dst_k.stride(0), dst_k.stride(1),
                                       dst_k.stride(2), dst_k.shape[1], _stream(pool_k.device)),
           "pdllm_compact_kept_rows")
    return dst_k, dst_v


def gather_kept_kv(pool_k, pool_v, chunk_slot, sel_chunk, keep_rows, k_per_seq, dst_k=None, dst_v=None):
    """pdllm_gather_kept_kv: the attended pool rows of each sequence, gathered
    contiguously -- [n_seq * k_max][b + 1][h_kv][d] tensors (new, or the
    given dst_k / dst_v), where sequence s's K_s (b + 1) rows start at slot
    s * k_max.  Returns (dst_k, dst_v)."""
    pool = make_pool(pool_k, pool_v)
    for t, name in ((chunk_slot, "chunk_slot"), (sel_chunk, "sel_chunk"), (keep_rows, "keep_rows")):
        _dense(t, name, torch.int32)
    n_seq, k_max = sel_chunk.shape
    b = keep_rows.shape[1]
    if len(k_per_seq) != n_seq or chunk_slot.numel() % n_seq or keep_rows.shape[0] != chunk_slot.numel():
        raise ValueError("page table shapes do not agree")
    if dst_k is None:
        shape = (max(n_seq * k_max, 1), b + 1, pool.h_kv, pool.d)
        dst_k = torch.empty(shape, dtype=pool_k.dtype, device=pool_k.device)
        dst_v = torch.empty(shape, dtype=pool_k.dtype, device=pool_k.device)
    ks = (ctypes.c_int32 * n_seq)(*[int(x) for x in k_per_seq])
    pt = PageTable(chunk_slot.data_ptr(), sel_chunk.data_ptr(), keep_rows.data_ptr(), ctypes.cast(ks, ctypes.c_void_p),
                   chunk_slot.numel() // n_seq, k_max, b, 0)
    _check(lib.pdllm_gather_kept_kv(ctypes.byref(pool), ctypes.byref(pt), n_seq, dst_k.data_ptr(), dst_v.data_ptr(),
                                    dst_k.stride(0), dst_k.stride(1), dst_k.stride(2), _stream(pool_k.device)),
           "pdllm_gather_kept_kv")
    return dst_k, dst_v


def decode_plan(k_per_seq, b, l_d, h_q, h_kv, d, dtype, num_splits=0, n_cu=256, with_rows=False):
    """pdllm_decode_plan (host only): returns (splits, tiles_per_split,
    workspace_bytes), and the query rows per workgroup if ``with_rows``."""
    n_seq = len(k_per_seq)
    ks = (ctypes.c_int32 * n_seq)(*[int(x) for x in k_per_seq])
    splits = (ctypes.c_int32 * n_seq)()
    tps = (ctypes.c_int32 * n_seq)()
    rows = ctypes.c_int32(0)
    ws = ctypes.c_int64(0)
    _check(lib.pdllm_decode_plan(ks, n_seq, b, l_d, h_q, h_kv, d, dtype, num_splits, n_cu, splits,
                                 tps, ctypes.byref(rows), ctypes.byref(ws)), "pdllm_decode_plan")
    if with_rows:
        return list(splits), list(tps), ws.value, rows.value
    return list(splits), list(tps), ws.value


class Decode:
    """A prepared pdllm_split_attn_decode call: the structs, host K_s array,
    outputs and workspace are built once so repeated calls (timing loops,
    denoising steps) only cross the boundary.  ``keep_rows`` is the
    [n_seq * N][b] table over a whole-chunk pool (-1 entries: absent rows of a
    partial chunk).  For a pool of compacted slots (pdllm_compact_kept_rows),
    whose kept rows are rows 1..b, pass ``compacted=True`` with ``keep_rows``
    (read only for its -1 entries) or with keep_rows=None and ``b``.
    ``q_rows_per_wg`` forces the workgroup shape and ``merge`` the merge
    (pdllm_decode_opts; 0 = the library's choice).  With ``resolve`` the
    attended pool rows are resolved once here (pdllm_resolve_rows, into
    ``self.rows``) and every call reads them instead of the index tables;
    call ``resolve()`` again after the tables change.  The workspace is
    zero-filled once, as the in-kernel merge requires."""

    def __init__(self, pool_k, pool_v, chunk_slot, sel_chunk, keep_rows, k_per_seq, q, k_resp,
                 v_resp, scale, num_splits=0, want_lse=True, out=None, b=None, compacted=False,
                 q_rows_per_wg=0, merge=0, resolve=False):
        self.pool = make_pool(pool_k, pool_v)
        compacted = compacted or keep_rows is None
        no_table = keep_rows is None
        if no_table:
            if b is None:
                raise ValueError("a compacted pool without keep_rows needs b")
            keep_rows = torch.empty((chunk_slot.numel(), int(b)), dtype=torch.int32, device=q.device)
        for t, name in ((chunk_slot, "chunk_slot"), (sel_chunk, "sel_chunk"), (keep_rows, "keep_rows")):
            _dense(t, name, torch.int32)
        _dense(q, "q", pool_k.dtype)
        _dense(k_resp, "k_resp", pool_k.dtype)
        _dense(v_resp, "v_resp", pool_k.dtype)
        n_seq, l_d, h_q, d = q.shape
        if d != self.pool.d or k_resp.shape != (n_seq, l_d, self.pool.h_kv, d) or v_resp.shape != k_resp.shape:
            raise ValueError("q / k_resp / v_resp shapes do not match the pool")
        if sel_chunk.dim() != 2 or sel_chunk.shape[0] != n_seq:
            raise ValueError("sel_chunk must be [n_seq][k_max]")
        if keep_rows.dim() != 2 or chunk_slot.numel() % n_seq or keep_rows.shape[0] != chunk_slot.numel():
            raise ValueError("keep_rows must be [n_seq * N][b] and chunk_slot [n_seq * N]")
        self._keep = (chunk_slot, sel_chunk, keep_rows, q, k_resp, v_resp, pool_k, pool_v)
        self.ks = (ctypes.c_int32 * n_seq)(*[int(x) for x in k_per_seq])
        self.pt = PageTable(chunk_slot.data_ptr(), sel_chunk.data_ptr(),
                            None if no_table else keep_rows.data_ptr(),
                            ctypes.cast(self.ks, ctypes.c_void_p), chunk_slot.numel() // n_seq,
                            sel_chunk.shape[1], keep_rows.shape[1], 1 if compacted else 0)
        self.n_seq, self.l_d, self.h_q = n_seq, l_d, h_q
        self.scale = float(scale)
        self.num_splits = int(num_splits)
        self.opts = DecodeOpts(int(num_splits), int(q_rows_per_wg), int(merge))
        dev = q.device
        self.device = dev
        self.o = out if out is not None else torch.empty_like(q)
        self.lse = torch.empty((n_seq, h_q, l_d), dtype=torch.float32, device=dev) if want_lse else None
        need = lib.pdllm_split_attn_decode_ex_workspace(ctypes.byref(self.pool), ctypes.byref(self.pt),
                                                        n_seq, l_d, h_q, ctypes.byref(self.opts))
        self.workspace = torch.zeros(max(int(need), 256), dtype=torch.uint8, device=dev)
        self.rows = None
        if resolve:
            self.rows = torch.empty(max(n_seq * self.pt.k_max * (self.pt.b + 1), 1), dtype=torch.int32, device=dev)
            self.resolve()

    def resolve(self, stream: Optional[int] = None):
        """pdllm_resolve_rows into ``self.rows`` (from the index tables), then
        point the page table at it."""
        self.pt.rows = None
        _check(lib.pdllm_resolve_rows(ctypes.byref(self.pool), ctypes.byref(self.pt), self.n_seq,
                                      self.rows.data_ptr(), self.rows.numel(),
                                      _stream(self.device) if stream is None else stream), "pdllm_resolve_rows")
        self.pt.rows = self.rows.data_ptr()

    def __call__(self, stream: Optional[int] = None):
        st = lib.pdllm_split_attn_decode_ex(
            ctypes.byref(self.pool), ctypes.byref(self.pt), self._keep[3].data_ptr(),
            self._keep[4].data_ptr(), self._keep[5].data_ptr(), self.n_seq, self.l_d, self.h_q,
            self.scale, ctypes.byref(self.opts), self.o.data_ptr(), _ptr(self.lse), self.workspace.data_ptr(),
            self.workspace.numel(), _stream(self.device) if stream is None else stream)
        _check(st, "pdllm_split_attn_decode_ex")
        return self.o, self.lse


def split_attn_decode(pool_k, pool_v, chunk_slot, sel_chunk, keep_rows, k_per_seq, q, k_resp,
                      v_resp, scale, num_splits=0, want_lse=True, b=None, compacted=False, q_rows_per_wg=0,
                      merge=0, resolve=False):
    """pdllm_split_attn_decode; returns (o [n_seq][L_d][h_q][d], lse [n_seq][h_q][L_d] or None).
    compacted=True (or keep_rows=None with ``b``) decodes over a pool of compacted slots."""
    return Decode(pool_k, pool_v, chunk_slot, sel_chunk, keep_rows, k_per_seq, q, k_resp, v_resp,
                  scale, num_splits, want_lse, b=b, compacted=compacted, q_rows_per_wg=q_rows_per_wg,
                  merge=merge, resolve=resolve)()
