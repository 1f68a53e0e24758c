"""Pins of the oracle on a prefix that ends in a partial chunk (a chunk of
C' < C tokens after its BOS; the pages cut the prefix into chunks of C
tokens and do not treat the remainder, so it is read as a shorter chunk),
independent of the oracle's own code:

* the partial chunk's prefill output against the library routine
  ``torch.nn.functional.scaled_dot_product_attention`` (fp64, CPU) over its
  first R_c rows, and its per-key scores against a loop-by-loop brute force;
  the slot rows past R_c hold large values, so any use of them shows;
* closed form: the scores of a chunk of R_c rows sum to W * h_q and its keys
  past R_c score 0;
* top-B against ``numpy.lexsort`` over the chunk's own content rows, with
  every row kept (then -1 entries) when it has fewer than B;
* decode with absent (-1) kept-row entries against the library attention
  over the explicitly gathered present rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _cfg(**kw):
    base = dict(name="pin", h_q=4, h_kv=2, d=8, dtype="f32", n_chunks=4, chunk=9,
                k_per_seq=(3,), b=5, l_d=5, w=3, n_seq=1, last_chunk=3)
    base.update(kw)
    return synth.Config(**base)


def _sdpa(q, k, v, scale, g_size):
    """q [rows][h_q][d], k/v [rows'][h_kv][d] float64 -> [rows][h_q][d]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g_size, dim=0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g_size, dim=0)[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("seed,kw", [(0, {}), (1, dict(n_seq=2, h_q=6, h_kv=3, last_chunk=1)),
                                     (2, dict(dtype="bf16", d=16, last_chunk=8))])
def test_partial_chunk_prefill_is_sdpa_over_its_rows(seed, kw):
    cfg = _cfg(**kw)
    inp = synth.generate(cfg, seed, with_q_chunk=True)
    rows = cfg.chunk_rows
    o, score = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                          cfg.n_chunks, cfg.scale, chunk_rows=rows)
    g_size = cfg.h_q // cfg.h_kv
    for c in range(cfg.n_slots):
        rc, slot = int(rows[c]), int(inp.chunk_slot[c])
        ref = _sdpa(oracle.as_f64(inp.q_chunk[c, :rc]), oracle.as_f64(inp.pool_k[slot, :rc]),
                    oracle.as_f64(inp.pool_v[slot, :rc]), cfg.scale, g_size)
        np.testing.assert_allclose(o[c, :rc], ref, rtol=0, atol=1e-12)
        assert np.isnan(o[c, rc:]).all()
        assert (score[c, rc:] == 0).all()
        assert abs(score[c].sum() - cfg.w * cfg.h_q) <= 1e-12 * cfg.w * cfg.h_q


def test_partial_chunk_scores_match_brute_force():
    cfg = _cfg(last_chunk=2, chunk=6)
    inp = synth.generate(cfg, 5, with_q_chunk=True)
    rows = cfg.chunk_rows
    _, score = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                          cfg.n_chunks, cfg.scale, chunk_rows=rows)
    pk, qw = oracle.as_f64(inp.pool_k), oracle.as_f64(inp.q_win)
    g_size = cfg.h_q // cfg.h_kv
    for c in range(cfg.n_slots):
        rc, slot = int(rows[c]), int(inp.chunk_slot[c])
        want = [0.0] * cfg.rows
        for h in range(cfg.h_q):
            for w in range(cfg.w):
                z = [cfg.scale * sum(qw[0, w, h, e] * pk[slot, j, h // g_size, e] for e in range(cfg.d))
                     for j in range(rc)]
                ex = [math.exp(t - max(z)) for t in z]
                for j in range(rc):
                    want[j] += ex[j] / sum(ex)
        np.testing.assert_allclose(score[c], want, rtol=0, atol=1e-12)


def _lexsort_top(values, candidates, count):
    vals = np.asarray([values[j] for j in candidates], dtype=np.float64)
    idx = np.asarray(candidates)
    order = np.lexsort((idx, -np.nan_to_num(vals, nan=0.0), np.isnan(vals)))   # NaN last, larger first
    return sorted(idx[order[:count]].tolist())


@pytest.mark.parametrize("b", [0, 2, 3, 6, 9])
def test_topb_of_a_partial_chunk(b):
    rng = np.random.default_rng(b)
    n_chunks, r = 5, 10
    score = rng.random((n_chunks, r)).astype(np.float32)
    score[1, 4] = score[1, 2]                       # a tie inside a partial chunk
    rows = np.array([10, 5, 1, 4, 10], dtype=np.int32)
    keep = oracle.select_topb(score, b, chunk_rows=rows)
    for c in range(n_chunks):
        n_c = int(rows[c]) - 1
        want = _lexsort_top(score[c], list(range(1, n_c + 1)), min(b, n_c))
        assert keep[c, :len(want)].tolist() == want
        assert (keep[c, len(want):] == -1).all()
        if b >= n_c:
            assert keep[c, :n_c].tolist() == list(range(1, n_c + 1))


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_skips_absent_rows(seed):
    cfg = _cfg(b=5, last_chunk=2, k_per_seq=(4,), n_chunks=4)  # K = N: the partial chunk is selected
    inp = synth.generate(cfg, seed)
    sel, keep = synth.random_page_table(cfg, seed)
    assert (keep == -1).any()
    o, lse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                      inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    # the attended rows, gathered by hand: BOS, then the present kept rows
    ks, vs = [], []
    for k in range(cfg.k_per_seq[0]):
        c = int(sel[0, k])
        slot = int(inp.chunk_slot[c])
        for r in [0] + [int(x) for x in keep[c] if x != -1]:
            ks.append(oracle.as_f64(inp.pool_k[slot, r]))
            vs.append(oracle.as_f64(inp.pool_v[slot, r]))
    kk = np.concatenate([np.stack(ks), oracle.as_f64(inp.k_resp[0])])
    vv = np.concatenate([np.stack(vs), oracle.as_f64(inp.v_resp[0])])
    n_present = sum(1 for c in sel[0] for x in keep[c] if x != -1)
    assert kk.shape[0] == cfg.k_per_seq[0] + n_present + cfg.l_d
    ref = _sdpa(oracle.as_f64(inp.q[0]), kk, vv, cfg.scale, cfg.h_q // cfg.h_kv)
    np.testing.assert_allclose(o[0], ref, rtol=0, atol=1e-12)
    assert np.isfinite(lse).all()


def test_chunk_rows_of_configs():
    assert (synth.config("s32").chunk_rows == 257).all()
    cfg = _cfg(n_seq=2)
    assert cfg.chunk_rows.tolist() == [10, 10, 10, 4, 10, 10, 10, 4]
