"""fp64 CPU oracle for the Prefilling-dLLM chunk-sparse attention path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in
``oracle/``.  The product path (``diffusion_long_context_amd``) never imports
it and shares no code with it; the two meet only through the seeded input
arrays of the ``synth`` module.

Every function computes the *plain definition* of one step, in float64, with
no blocking, fusion or reordering beyond what the definition states.  numpy's
``@`` (matrix product), ``exp``, ``max`` and ``sum`` serve as library
primitives.  Sources are the technical summary pages of "Prefilling-dLLM:
Predictive Prefilling for Long-Context Inference in Diffusion Language
Models" (gist.science, paper 2606.10537); section names refer to that
summary:

* Methodology, "1. Chunked prefill and KV cache": the prefix is cut into N
  chunks of C tokens, each gets a BOS token prepended, and each chunk is run
  with bidirectional attention restricted to itself; the top-K chunks by a
  given score s are selected.
* Methodology, "2. Two-level sparsity": only the K selected chunks take part
  in decode attention, and inside each of them only the B tokens with the
  largest cumulative bidirectional attention weight from the query tokens are
  kept.
* Methodology, "3. Decoding with static KV reuse": the cached chunk KV stays
  fixed across denoising steps; only the query / response rows' KV is
  recomputed, and the decode rows attend to both.
* "Attention kernel optimization": the decode attention may be split along
  the KV dimension into independent parts that are merged by a log-sum-exp
  reduction (``lse_merge`` below is that merge, used to pin split
  invariance).
* Methodology 1, predictive scoring: each chunk is scored by the negative
  log-likelihood of the query window given the chunk (s_I) and by the
  likelihood of the pseudo-labels given the chunk and the query (s_P), and
  s = s_I + s_P feeds the top-K (``chunk_scores``).

Readings where the pages are silent (each is listed with its support in the
design notes):
  * BOS (row 0 of a chunk slot) is always kept and attended; top-B ranks the
    C content rows 1..C only, so a selected chunk contributes B + 1 rows.
  * The scoring window's softmax is normalised over the chunk's own R = C + 1
    keys only, and a key's score is the plain sum of its softmax weight over
    all query heads and all window rows.
  * No mask anywhere (bidirectional); positions are already applied to Q, K.
  * Query head h reads KV head floor(h / G), G = h_q / h_kv (grouped query
    attention with G consecutive query heads per KV head).
  * Selection order: larger score first, ties to the lower index, -0 == +0,
    NaN after every number; the kept indices are returned in ascending order.
  * lse is the natural logarithm of the softmax normaliser (with max).
  * s_P's "likelihood" is read as a log-likelihood (a sum of per-token
    log-probabilities), the only reading that can be added to the
    negative log-likelihood s_I; both are natural-log sums over the
    vocabulary-wide softmax of each scored row.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# input decoding
# --------------------------------------------------------------------------
def as_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of a float32 array or of bf16 bit patterns (uint16).

    A bfloat16 number is the top half of a float32, so shifting its 16 bits
    into the high half of a 32-bit word gives the same value as a float32,
    which widens exactly to float64.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head h when ``group`` query heads share a KV head."""
    return h // group


def softmax_rows(z: np.ndarray):
    """Row-wise softmax in two passes: subtract the row max, exponentiate,
    divide by the row sum.  Returns (p, m, l) with m the row max and l the sum
    of exp(z - m), so that the row's log-normaliser is m + ln l."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    l = np.sum(e, axis=-1, keepdims=True)
    return e / l, m[..., 0], l[..., 0]


# --------------------------------------------------------------------------
# prefill side: chunk-local attention and per-key scoring
# --------------------------------------------------------------------------
def chunk_prefill_score(pool_k, pool_v, chunk_slot, q_chunk, q_win, chunks_per_win,
                        scale, chunks: Optional[Sequence[int]] = None, chunk_rows=None):
    """Chunk-local bidirectional attention plus per-key cumulative weight.

    Methodology 1 (each chunk, BOS first, attends only to itself) and
    Methodology 2 (intra-chunk sparsity ranks a chunk's tokens by their
    cumulative bidirectional attention weight from the query tokens).

    pool_k, pool_v : [n_slots][R][h_kv][d]; chunk c lives in slot chunk_slot[c]
    q_chunk        : [n_chunks][R][h_q][d]   the chunk's own queries
    q_win          : [n_win][W][h_q][d]      chunk c is scored by window
                                             c // chunks_per_win
    chunk_rows     : optional [n_chunks] rows held by each chunk (default R).
                     A prefix whose length is not a multiple of C ends in a
                     partial chunk: its BOS and the C' < C remaining tokens,
                     R_c = C' + 1 rows at the start of its slot.
    Returns (o_chunk [len(chunks)][R][h_q][d], key_score [len(chunks)][R]),
    both float64, for ``chunks`` (default: all chunks, in order).

    o_chunk[c, r, h]  = sum_j softmax_j(scale <Qc[c,r,h], K[slot,j,g]>) V[slot,j,g]
    key_score[c, j]   = sum_h sum_w softmax_j(scale <Qw[w,h], K[slot,j,g]>)
    with g = kv_head_of(h, G) and r, j over the chunk's R_c rows: a partial
    chunk is a chunk of R_c rows.  Its output rows r >= R_c are not defined
    (NaN here) and its keys j >= R_c score 0.
    """
    n_chunks = q_chunk.shape[0]
    _, r_rows, h_kv, _ = pool_k.shape
    h_q = q_chunk.shape[2]
    group = h_q // h_kv
    if chunks is None:
        chunks = range(n_chunks)
    chunks = list(chunks)
    d = pool_k.shape[3]
    o = np.zeros((len(chunks), r_rows, h_q, d))
    score = np.zeros((len(chunks), r_rows))
    for n, c in enumerate(chunks):
        slot = int(chunk_slot[c])
        rc = r_rows if chunk_rows is None else int(chunk_rows[c])
        kk = as_f64(pool_k[slot, :rc])     # [R_c][h_kv][d]
        vv = as_f64(pool_v[slot, :rc])
        qc = as_f64(q_chunk[c, :rc])       # [R_c][h_q][d]
        qw = as_f64(q_win[c // chunks_per_win])   # [W][h_q][d]
        o[n, rc:] = np.nan
        for h in range(h_q):
            g = kv_head_of(h, group)
            k_g, v_g = kk[:, g, :], vv[:, g, :]
            p, _, _ = softmax_rows(scale * (qc[:, h, :] @ k_g.T))      # [R_c][R_c]
            o[n, :rc, h, :] = p @ v_g
            pw, _, _ = softmax_rows(scale * (qw[:, h, :] @ k_g.T))     # [W][R_c]
            score[n, :rc] += pw.sum(axis=0)
    return o, score


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------
def _rank_key(value: float, index: int):
    """Sort key of the selection order: larger first, NaN last, then index."""
    if math.isnan(value):
        return (1, 0.0, index)
    return (0, -value, index)


def _top(values: np.ndarray, candidates: Sequence[int], count: int) -> List[int]:
    order = sorted(candidates, key=lambda j: _rank_key(float(values[j]), j))
    return sorted(order[:count])


def select_topb(key_score: np.ndarray, b: int, chunk_rows=None) -> np.ndarray:
    """Top-B content rows of every chunk (Methodology 2, intra-chunk sparsity).

    key_score  : [n_chunks][R] (float32 as the GPU holds it, or float64)
    chunk_rows : optional [n_chunks] rows held by each chunk (default R)
    Returns keep_rows [n_chunks][b] int32: the b best rows among 1..R_c-1 (row
    0 is the BOS anchor, always kept and not a candidate), ascending.  A
    partial chunk with fewer than b content rows keeps all of them, and the
    rest of its entries are -1 (absent).
    """
    n_chunks, r_rows = key_score.shape
    out = np.full((n_chunks, b), -1, dtype=np.int32)
    for c in range(n_chunks):
        rc = r_rows if chunk_rows is None else int(chunk_rows[c])
        kept = _top(key_score[c], range(1, rc), min(b, rc - 1))
        out[c, :len(kept)] = kept
    return out


def select_topk(chunk_score: np.ndarray, k_per_seq: Sequence[int], k_max: int) -> np.ndarray:
    """Top-K chunks of every sequence by the given score s (Methodology 1,
    selection; Methodology 2, inter-chunk sparsity).

    chunk_score : [n_seq][N];  k_per_seq[s] = K_s <= k_max
    Returns sel_chunk [n_seq][k_max] int32: the K_s best chunk ids in
    ascending order, then -1 padding.
    """
    n_seq, n = chunk_score.shape
    out = np.full((n_seq, k_max), -1, dtype=np.int32)
    for s in range(n_seq):
        ks = int(k_per_seq[s])
        out[s, :ks] = _top(chunk_score[s], range(n), ks)
    return out


# --------------------------------------------------------------------------
# decode: attention over the kept chunk rows plus the response rows
# --------------------------------------------------------------------------
def attended_pool_rows(chunk_slot, sel_chunk, keep_rows, k_s: int, seq: int,
                       n_chunks_per_seq: int) -> Tuple[np.ndarray, np.ndarray]:
    """(slot, row) of every cached row sequence ``seq`` attends to, in chunk
    order: for each selected chunk, BOS row 0 then its kept rows (absent
    entries, -1, of a partial chunk are skipped)."""
    slots, rows = [], []
    for k in range(k_s):
        c = seq * n_chunks_per_seq + int(sel_chunk[seq][k])
        slot = int(chunk_slot[c])
        for r in [0] + [int(x) for x in keep_rows[c] if x >= 0]:
            slots.append(slot)
            rows.append(r)
    return np.asarray(slots, dtype=np.int64), np.asarray(rows, dtype=np.int64)


def compact_kept_rows(pool_k, pool_v, chunk_slot, keep_rows, n_chunks: int):
    """Kept-row cache of the first ``n_chunks`` chunks (Methodology 2: after
    the intra-chunk selection only a chunk's top-B tokens stay in the KV
    cache; the BOS anchor stays with them).

    pool_k, pool_v : [n_slots][R][h_kv][d];  keep_rows : [n_chunks][b]
    Returns (k, v, written): [n_slots][b + 1][h_kv][d] arrays of the pool's
    dtype where slot s = chunk_slot[c] holds the chunk's BOS row, then its
    kept rows in keep_rows order; ``written`` [n_slots][b + 1] flags the rows
    that hold a row of a chunk (the others are zero): an absent entry (-1) of
    a partial chunk writes nothing.
    """
    n_slots, _, h_kv, d = pool_k.shape
    b = keep_rows.shape[1]
    k = np.zeros((n_slots, b + 1, h_kv, d), dtype=pool_k.dtype)
    v = np.zeros_like(k)
    written = np.zeros((n_slots, b + 1), dtype=bool)
    for c in range(n_chunks):
        slot = int(chunk_slot[c])
        for j, r in enumerate([0] + [int(x) for x in keep_rows[c]]):
            if r < 0:
                continue
            k[slot, j] = pool_k[slot, r]
            v[slot, j] = pool_v[slot, r]
            written[slot, j] = True
    return k, v, written


def all_rows_kept(n_chunks: int, b: int) -> np.ndarray:
    """The keep_rows table of compacted slots: chunk c's kept rows are rows
    1..b of its slot ([n_chunks][b] int32)."""
    return np.tile(np.arange(1, b + 1, dtype=np.int32), (n_chunks, 1))


def attended_kv(pool_k, pool_v, chunk_slot, sel_chunk, keep_rows, k_s, seq,
                n_chunks_per_seq, k_resp, v_resp):
    """Dense [N_kv][h_kv][d] float64 keys and values attended by ``seq``:
    the kept pool rows (static cache, Methodology 3) followed by the L_d
    recomputed response rows."""
    slots, rows = attended_pool_rows(chunk_slot, sel_chunk, keep_rows, k_s, seq,
                                     n_chunks_per_seq)
    kp = as_f64(pool_k[slots, rows]) if len(slots) else np.zeros((0,) + pool_k.shape[2:])
    vp = as_f64(pool_v[slots, rows]) if len(slots) else np.zeros((0,) + pool_v.shape[2:])
    kk = np.concatenate([kp, as_f64(k_resp[seq])], axis=0)
    vv = np.concatenate([vp, as_f64(v_resp[seq])], axis=0)
    return kk, vv


def split_attn_decode(pool_k, pool_v, chunk_slot, sel_chunk, keep_rows, k_per_seq,
                      q, k_resp, v_resp, scale, heads: Optional[Sequence[int]] = None):
    """Decode-step attention of the L_d window rows (Methodology 2 and 3).

    For sequence s, token i and query head h, the attended set A_s is every
    selected chunk's BOS row and kept rows plus the L_d response rows; the
    output is the softmax-weighted mean of their values:
        z_a = scale <q[s,i,h], k_a[g]>,  o = sum_a softmax(z)_a v_a[g],
        lse = ln sum_a exp(z_a).
    Returns (o [n_seq][L_d][h_q][d], lse [n_seq][h_q][L_d]) float64; heads not
    in ``heads`` (default: all) are left as NaN.
    """
    n_seq, l_d, h_q, d = q.shape
    h_kv = k_resp.shape[2]
    group = h_q // h_kv
    n_per_seq = len(chunk_slot) // n_seq
    heads = range(h_q) if heads is None else heads
    o = np.full((n_seq, l_d, h_q, d), np.nan)
    lse = np.full((n_seq, h_q, l_d), np.nan)
    for s in range(n_seq):
        kk, vv = attended_kv(pool_k, pool_v, chunk_slot, sel_chunk, keep_rows,
                             int(k_per_seq[s]), s, n_per_seq, k_resp, v_resp)
        qs = as_f64(q[s])
        for h in heads:
            g = kv_head_of(h, group)
            p, m, l = softmax_rows(scale * (qs[:, h, :] @ kk[:, g, :].T))
            o[s, :, h, :] = p @ vv[:, g, :]
            lse[s, h, :] = m + np.log(l)
    return o, lse


# --------------------------------------------------------------------------
# split-KV with log-sum-exp merge (used to pin split invariance)
# --------------------------------------------------------------------------
def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge per-part attention results ("Attention kernel optimization").

    o_parts [S][..., d] are per-part normalised outputs and lse_parts [S][...]
    their log-normalisers (an empty part has lse = -inf and any o).  With
    M = max_s lse_s:  lse = M + ln sum_s exp(lse_s - M),
    o = sum_s exp(lse_s - lse) o_s.
    """
    m = np.max(lse_parts, axis=0)
    w = np.exp(lse_parts - m[None])                    # -inf parts weigh 0
    total = np.sum(w, axis=0)
    lse = m + np.log(total)
    wn = w / total[None]
    o = np.sum(np.where(wn[..., None] > 0, wn[..., None] * o_parts, 0.0), axis=0)
    return o, lse


def attention_over_parts(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                         scale: float, parts: Sequence[np.ndarray]):
    """Attention of q_rows [M][d] over k_rows/v_rows [N][d] computed on each
    part (an index array into the N rows) separately, then LSE-merged."""
    m_rows, d = q_rows.shape
    o_parts = np.zeros((len(parts), m_rows, d))
    lse_parts = np.full((len(parts), m_rows), -np.inf)
    for i, idx in enumerate(parts):
        if len(idx) == 0:
            continue
        p, m, l = softmax_rows(scale * (q_rows @ k_rows[idx].T))
        o_parts[i] = p @ v_rows[idx]
        lse_parts[i] = m + np.log(l)
    return lse_merge(o_parts, lse_parts)


# --------------------------------------------------------------------------
# chunk scores from per-token log-probabilities
# --------------------------------------------------------------------------
def token_log_probs(logits: np.ndarray, target: np.ndarray) -> np.ndarray:
    """Log-probability of each row's target token: logits [n][V] (bf16 bits or
    float32), target [n] ids in [0, V) -> [n] float64, with
    log p = z[target] - ln sum_v exp(z[v])  (the row's log-softmax at the
    target; the sum is taken against the row maximum)."""
    z = as_f64(logits).reshape(-1, logits.shape[-1])
    t = np.asarray(target).reshape(-1)
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return z[np.arange(z.shape[0]), t] - lse


def chunk_scores(logits: np.ndarray, target: np.ndarray, n_query: int, n_pseudo: int):
    """Predictive chunk scores (Methodology 1, predictive scoring), from the
    model's logits at each chunk's scored positions:

    logits [n_chunks][n_query + n_pseudo][V]: rows 0..n_query-1 predict the
    query window's tokens, the next n_pseudo rows the pseudo-label tokens;
    target [n_chunks][n_query + n_pseudo] holds those token ids.

    s_I = -sum over the query rows of log p   (negative log-likelihood of the
          query window given the chunk)
    s_P =  sum over the pseudo-label rows of log p   (log-likelihood of the
          pseudo-labels given the chunk and the query)
    s   = s_I + s_P
    Returns (s_i, s_p, s), each float64 [n_chunks]; rows summed in order.
    """
    n_chunks = logits.shape[0]
    lp = token_log_probs(logits, target).reshape(n_chunks, n_query + n_pseudo)
    s_i = -lp[:, :n_query].sum(axis=1)
    s_p = lp[:, n_query:].sum(axis=1)
    return s_i, s_p, s_i + s_p
