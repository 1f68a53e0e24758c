"""Seeded synthetic inputs for the chunk-sparse attention path.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no attention, no softmax, no selection).  Both the fp64
oracle (``oracle/``) and the HIP path (``diffusion_long_context_amd``) are fed
from the arrays it returns, so that the two sides see bit-identical inputs.

Shapes follow the Prefilling-dLLM summary (gist.science, paper 2606.10537):
the prefix is cut into N non-overlapping chunks of C tokens with a BOS token
prepended to each (Methodology, "1. Chunked prefill and KV cache"), so one
cached chunk occupies R = C + 1 rows.  The chunk KV lives in a pool of slots
in a random order, i.e. non-contiguously ("Attention kernel optimization").

Layouts (row-major, last index fastest):
  pool_k, pool_v  [n_slots][R][h_kv][d]   slot chunk_slot[c] holds chunk c
  chunk_slot      [n_seq*N]  int32         a permutation of the slots
  chunk_score     [n_seq][N] float32       given per-chunk scores, distinct
  q               [n_seq][L_d][h_q][d]     decode-window queries
  k_resp, v_resp  [n_seq][L_d][h_kv][d]    recomputed response keys/values
  q_chunk         [n_seq*N][R][h_q][d]     each chunk's own prefill queries
  q_win           [n_seq][W][h_q][d]       query window used to score keys

Floating data is drawn in float32 and, for bf16 configurations, rounded once
to bfloat16 (round-to-nearest-even); bf16 arrays are returned as their uint16
bit patterns.

Draw order for one seed (numpy PCG64 ``default_rng(seed)``):
  1 pool permutation, 2 chunk scores, 3 pool K (+ per-chunk key offsets),
  4 pool V, 5 q, 6 k_resp, 7 v_resp, 8 q_chunk (only when requested).
The query window is the first W rows of ``q`` of the chunk's own sequence.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np


@dataclass(frozen=True)
class Config:
    """One synthetic workload.  Sizes are in tokens / rows / heads."""

    name: str
    h_q: int
    h_kv: int
    d: int
    dtype: str                 # "f32" or "bf16"
    n_chunks: int              # N chunks per sequence
    chunk: int                 # C content tokens per chunk (R = C + 1 rows)
    k_per_seq: tuple           # K_s selected chunks per sequence
    b: int                     # B kept content rows per chunk
    l_d: int                   # decode-window rows (query + response)
    w: int                     # query-window rows used to score keys
    n_seq: int = 1
    key_offset_std: float = 0.0  # per-(chunk, kv head) key-mean offset std
    key_dist: str = "normal"     # "normal" or "t4" (Student-t, 4 dof)
    layers: int = 1
    steps: int = 1
    last_chunk: int = 0          # tokens of each sequence's last chunk (0: C, a full chunk)

    @property
    def rows(self) -> int:
        return self.chunk + 1

    @property
    def n_slots(self) -> int:
        return self.n_seq * self.n_chunks

    @property
    def chunk_rows(self) -> np.ndarray:
        """[n_seq*N] int32 rows held by each chunk: R, except a partial last
        chunk of each sequence (BOS + last_chunk tokens)."""
        rows = np.full((self.n_seq, self.n_chunks), self.rows, dtype=np.int32)
        if self.last_chunk:
            rows[:, -1] = self.last_chunk + 1
        return rows.reshape(-1)

    @property
    def k_max(self) -> int:
        return max(self.k_per_seq) if self.k_per_seq else 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


CONFIGS: Dict[str, Config] = {
    # 1/1 heads, d=64, fp32, 512-token prefix = 8 chunks of 64 (+BOS), K=2,
    # B=16, 32 decode rows that also form the scoring window.
    "tiny": Config("tiny", 1, 1, 64, "f32", 8, 64, (2,), 16, 32, 32),
    # Dream-7B-like GQA 28/4, d=128, bf16, 8K prefix, K=8, B=128, L_d=256,
    # per-chunk key-mean offset N(0, 0.5).
    "s8": Config("s8", 28, 4, 128, "bf16", 32, 256, (8,), 128, 256, 64,
                 key_offset_std=0.5),
    # 32K prefix, K=16, B=256 (whole chunks kept), L_d=256.
    "s32": Config("s32", 28, 4, 128, "bf16", 128, 256, (16,), 256, 256, 64),
    # 128K prefix, batch 4 with K_s in {8,16,24,32}, B=128, L_d=512,
    # Student-t(4) keys.
    "s128": Config("s128", 28, 4, 128, "bf16", 512, 256, (8, 16, 24, 32), 128,
                   512, 64, n_seq=4, key_dist="t4"),
    # Full denoising run at 32K: 28 layers x 64 steps, K=16, B=128, L_d=256,
    # scoring window of 64 query rows.
    "f32": Config("f32", 28, 4, 128, "bf16", 128, 256, (16,), 128, 256, 64,
                  layers=28, steps=64),
}


def config(name: str, **overrides) -> Config:
    """Return a named configuration, optionally with fields replaced."""
    base = CONFIGS[name]
    return replace(base, **overrides) if overrides else base


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x)


def _keys(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "t4":
        return rng.standard_t(4, size=shape).astype(np.float32)
    raise ValueError(f"unknown key distribution {dist!r}")


def _distinct_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    """U(0,1) float32 draws, redrawn as a whole until all values differ."""
    n = int(np.prod(shape))
    while True:
        x = rng.random(n, dtype=np.float32)
        if np.unique(x).size == n:
            return x.reshape(shape)


@dataclass
class Inputs:
    cfg: Config
    seed: int
    chunk_slot: np.ndarray
    chunk_score: np.ndarray
    pool_k: np.ndarray
    pool_v: np.ndarray
    q: np.ndarray
    k_resp: np.ndarray
    v_resp: np.ndarray
    q_chunk: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def q_win(self) -> np.ndarray:
        """[n_seq][W][h_q][d]: the first W decode rows of each sequence."""
        return np.ascontiguousarray(self.q[:, : self.cfg.w])

    def sha256(self) -> Dict[str, str]:
        out = {}
        for name in ("chunk_slot", "chunk_score", "pool_k", "pool_v", "q",
                     "k_resp", "v_resp", "q_chunk"):
            a = getattr(self, name)
            if a is not None:
                out[name] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
        return out


def generate(cfg: Config, seed: int = 0, with_q_chunk: bool = False) -> Inputs:
    """Draw one workload's inputs in the documented order."""
    rng = np.random.default_rng(seed)
    n_slots, r, hk, hq, d = cfg.n_slots, cfg.rows, cfg.h_kv, cfg.h_q, cfg.d
    # 1. where each chunk's KV sits in the pool (one global permutation)
    chunk_slot = rng.permutation(n_slots).astype(np.int32)
    # 2. given per-chunk scores, distinct within each sequence
    chunk_score = _distinct_uniform(rng, (cfg.n_seq, cfg.n_chunks))
    # 3. pool keys, plus a per-(chunk, kv head) mean offset shared by the
    #    chunk's R rows; the offset is indexed by slot (a slot is one chunk)
    pk = _keys(rng, (n_slots, r, hk, d), cfg.key_dist)
    if cfg.key_offset_std > 0.0:
        off = rng.standard_normal((n_slots, 1, hk, d), dtype=np.float32)
        pk += np.float32(cfg.key_offset_std) * off
    pool_k = _finish(pk, cfg.dtype)
    del pk
    # 4. pool values
    pool_v = _finish(rng.standard_normal((n_slots, r, hk, d), dtype=np.float32), cfg.dtype)
    # 5-7. decode window queries and recomputed response keys / values
    q = _finish(rng.standard_normal((cfg.n_seq, cfg.l_d, hq, d), dtype=np.float32), cfg.dtype)
    k_resp = _finish(_keys(rng, (cfg.n_seq, cfg.l_d, hk, d), cfg.key_dist), cfg.dtype)
    v_resp = _finish(rng.standard_normal((cfg.n_seq, cfg.l_d, hk, d), dtype=np.float32), cfg.dtype)
    inp = Inputs(cfg, seed, chunk_slot, chunk_score, pool_k, pool_v, q, k_resp, v_resp)
    # 8. each chunk's own prefill queries (large: only on request)
    if with_q_chunk:
        inp.q_chunk = _finish(
            rng.standard_normal((n_slots, r, hq, d), dtype=np.float32), cfg.dtype)
    # A partial last chunk holds last_chunk + 1 rows; the rest of its slot
    # (and of its queries) is filled with large values, drawn from nothing,
    # so that any use of those rows shows in the results.
    if cfg.last_chunk:
        keep_rows = cfg.last_chunk + 1
        big_k, big_v = _finish(np.float32([30.0]), cfg.dtype)[0], _finish(np.float32([1000.0]), cfg.dtype)[0]
        for c in np.flatnonzero(cfg.chunk_rows < r):
            slot = int(chunk_slot[c])
            pool_k[slot, keep_rows:] = big_k
            pool_v[slot, keep_rows:] = big_v
            if inp.q_chunk is not None:
                inp.q_chunk[c, keep_rows:] = big_k
    return inp


def random_page_table(cfg: Config, seed: int = 0):
    """A seeded random but valid page table for decode-only cases.

    Returns ``(sel_chunk [n_seq][k_max] int32, keep_rows [n_seq*N][B] int32)``:
    each sequence's first K_s entries of ``sel_chunk`` are distinct chunk ids
    in ascending order, the rest are -1; each row of ``keep_rows`` holds B
    distinct content rows from 1..C in ascending order (a partial last chunk
    with fewer than B content rows: all of them, then -1).
    """
    rng = np.random.default_rng(1_000_003 + seed)
    k_max = cfg.k_max
    sel = np.full((cfg.n_seq, max(k_max, 0)), -1, dtype=np.int32)
    for s, ks in enumerate(cfg.k_per_seq):
        sel[s, :ks] = np.sort(rng.choice(cfg.n_chunks, size=ks, replace=False))
    keep = np.full((cfg.n_slots, cfg.b), -1, dtype=np.int32)
    rows = cfg.chunk_rows
    for c in range(cfg.n_slots):
        n_c = int(rows[c]) - 1               # content rows of the chunk
        count = min(cfg.b, n_c)
        keep[c, :count] = np.sort(rng.choice(np.arange(1, n_c + 1), size=count, replace=False))
    return sel, keep


def chunk_logits(n_chunks: int, n_query: int, n_pseudo: int, vocab: int, seed: int = 0,
                 dtype: str = "bf16", std: float = 2.5, stride: int = 0):
    """Seeded stand-in for the model's logits at each chunk's scored rows.

    Returns ``(logits [n_chunks][n_query + n_pseudo][stride or vocab], target
    [n_chunks][n_query + n_pseudo] int32)``: logits ~ N(0, std) drawn in
    float32 (rounded once to bf16 bits for ``dtype="bf16"``), padding columns
    past ``vocab`` set to 0; targets uniform over the vocabulary.  Half of the
    rows get their target logit raised by 2 std, so that the log-probabilities
    spread the way a model's do.
    """
    rng = np.random.default_rng(2_000_003 + seed)
    rows = n_query + n_pseudo
    width = max(stride, vocab)
    z = np.zeros((n_chunks, rows, width), dtype=np.float32)
    z[..., :vocab] = rng.normal(0.0, std, size=(n_chunks, rows, vocab)).astype(np.float32)
    target = rng.integers(0, vocab, size=(n_chunks, rows)).astype(np.int32)
    lift = rng.random((n_chunks, rows)) < 0.5
    ci, ri = np.nonzero(lift)
    z[ci, ri, target[ci, ri]] += np.float32(2.0 * std)
    return _finish(z, dtype), target


__all__ = ["Config", "CONFIGS", "config", "Inputs", "generate",
           "random_page_table", "f32_to_bf16_bits", "chunk_logits"]
