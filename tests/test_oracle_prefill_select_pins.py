"""Pins of the oracle's prefill attention, per-key scoring and selection:

* prefill output against the library routine
  ``torch.nn.functional.scaled_dot_product_attention`` (fp64, CPU) per chunk,
* brute force with explicit loops for the per-key score on tiny inputs,
* closed forms: the scores of a chunk sum to W * h_q (each window row's
  softmax sums to one); identical keys give every key W * h_q / R,
* a head-mapping probe: each KV head concentrates all of its query heads'
  weight on its own key, which a wrong query-head -> KV-head map misplaces,
* selection against ``numpy.lexsort`` (a library sort with the same order)
  on engineered arrays with ties, signed zeros, infinities and NaN.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _cfg(**kw):
    base = dict(name="pin", h_q=4, h_kv=2, d=8, dtype="f32", n_chunks=4, chunk=7,
                k_per_seq=(2,), b=3, l_d=5, w=3, n_seq=1)
    base.update(kw)
    return synth.Config(**base)


def _prefill(inp, cfg, q_chunk=None):
    qc = inp.q_chunk if q_chunk is None else q_chunk
    return oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, qc, inp.q_win,
                                      cfg.n_chunks, cfg.scale)


@pytest.mark.parametrize("seed,kw", [(0, {}), (1, dict(n_seq=2, h_q=6, h_kv=3)),
                                     (2, dict(dtype="bf16", d=16, chunk=5))])
def test_prefill_output_is_per_chunk_sdpa(seed, kw):
    cfg = _cfg(**kw)
    inp = synth.generate(cfg, seed, with_q_chunk=True)
    o, _ = _prefill(inp, cfg)
    g_size = cfg.h_q // cfg.h_kv
    for c in range(cfg.n_slots):
        slot = inp.chunk_slot[c]
        q = torch.from_numpy(oracle.as_f64(inp.q_chunk[c])).permute(1, 0, 2)[None]
        k = torch.from_numpy(oracle.as_f64(inp.pool_k[slot])).permute(1, 0, 2)
        v = torch.from_numpy(oracle.as_f64(inp.pool_v[slot])).permute(1, 0, 2)
        k = k.repeat_interleave(g_size, dim=0)[None]
        v = v.repeat_interleave(g_size, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=cfg.scale)
        np.testing.assert_allclose(o[c], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def _brute_scores(inp, cfg):
    pk = oracle.as_f64(inp.pool_k)
    qw = oracle.as_f64(inp.q_win)
    g_size = cfg.h_q // cfg.h_kv
    out = np.zeros((cfg.n_slots, cfg.rows))
    for c in range(cfg.n_slots):
        slot = inp.chunk_slot[c]
        win = qw[c // cfg.n_chunks]
        for h in range(cfg.h_q):
            g = h // g_size
            for w in range(cfg.w):
                z = [cfg.scale * sum(win[w, h, e] * pk[slot, j, g, e] for e in range(cfg.d))
                     for j in range(cfg.rows)]
                zmax = max(z)
                ex = [math.exp(t - zmax) for t in z]
                tot = sum(ex)
                for j in range(cfg.rows):
                    out[c, j] += ex[j] / tot
    return out


@pytest.mark.parametrize("seed,kw", [(0, {}), (3, dict(n_seq=2, w=2)), (4, dict(h_q=3, h_kv=1))])
def test_scores_match_brute_force(seed, kw):
    cfg = _cfg(**kw)
    inp = synth.generate(cfg, seed, with_q_chunk=True)
    _, score = _prefill(inp, cfg)
    np.testing.assert_allclose(score, _brute_scores(inp, cfg), rtol=0, atol=1e-12)


def test_scores_sum_to_window_rows_times_heads():
    cfg = _cfg(n_seq=2, w=4, h_q=6, h_kv=2)
    inp = synth.generate(cfg, 5, with_q_chunk=True)
    _, score = _prefill(inp, cfg)
    np.testing.assert_allclose(score.sum(axis=1), cfg.w * cfg.h_q, rtol=0, atol=1e-12)


def test_identical_keys_give_uniform_scores_and_mean_values():
    cfg = _cfg(h_q=4, h_kv=2, w=3)
    inp = synth.generate(cfg, 6, with_q_chunk=True)
    inp.pool_k[:] = inp.pool_k[0, 0]
    o, score = _prefill(inp, cfg)
    np.testing.assert_allclose(score, cfg.w * cfg.h_q / cfg.rows, rtol=0, atol=1e-12)
    # all-equal scores: the tie rule keeps the lowest content rows
    keep = oracle.select_topb(score.astype(np.float32), cfg.b)
    np.testing.assert_array_equal(keep, np.tile(np.arange(1, cfg.b + 1), (cfg.n_slots, 1)))
    g_size = cfg.h_q // cfg.h_kv
    pv = oracle.as_f64(inp.pool_v)
    for c in range(cfg.n_slots):
        for h in range(cfg.h_q):
            mean = pv[inp.chunk_slot[c], :, h // g_size].mean(0)
            np.testing.assert_allclose(o[c, :, h], np.broadcast_to(mean, o[c, :, h].shape),
                                       rtol=0, atol=1e-12)


def test_head_mapping_probe():
    """KV head g has one key aligned with every query; the window's weight of
    the G query heads reading g lands on that key.  Key j*_g = 1 + 2g."""
    cfg = _cfg(h_q=6, h_kv=3, d=8, chunk=7, w=2, n_chunks=1)
    inp = synth.generate(cfg, 0, with_q_chunk=True)
    u = np.zeros(cfg.d, dtype=np.float32)
    u[0] = 1.0
    inp.q[:] = u                                   # every window query = u
    inp.pool_k[:] = 0.0
    g_size = cfg.h_q // cfg.h_kv
    for g in range(cfg.h_kv):
        inp.pool_k[:, 1 + 2 * g, g, 0] = 400.0     # scale * 400 = ~141 logits
    _, score = _prefill(inp, cfg)
    for g in range(cfg.h_kv):
        assert abs(score[0, 1 + 2 * g] - cfg.w * g_size) < 1e-9
    assert abs(score[0].sum() - cfg.w * cfg.h_q) < 1e-9


# ------------------------------------------------------------------ selection
def _lexsort_top(values, candidates, count):
    vals = np.asarray(values, dtype=np.float64)[candidates]
    order = np.lexsort((np.asarray(candidates), -vals))    # NaN sorts last
    return np.sort(np.asarray(candidates)[order[:count]])


@pytest.mark.parametrize("seed", range(6))
def test_topb_matches_lexsort(seed):
    rng = np.random.default_rng(seed)
    n_chunks, r_rows = 5, 33
    ks = rng.integers(0, 6, size=(n_chunks, r_rows)).astype(np.float32)   # many ties
    if seed % 2:
        ks += rng.standard_normal(ks.shape).astype(np.float32)
    for b in (0, 1, 7, 16, 32):
        keep = oracle.select_topb(ks, b)
        for c in range(n_chunks):
            np.testing.assert_array_equal(keep[c], _lexsort_top(ks[c], list(range(1, r_rows)), b))


def test_topb_special_values():
    ks = np.array([[9.0, 0.0, -0.0, np.nan, np.inf, -np.inf, 1.0, 0.0, np.nan]], dtype=np.float32)
    # order over rows 1..8: inf(4), 1.0(6), 0.0(1), -0.0(2), 0.0(7), -inf(5), nan(3), nan(8)
    expect = {1: [4], 2: [4, 6], 3: [1, 4, 6], 4: [1, 2, 4, 6], 5: [1, 2, 4, 6, 7],
              6: [1, 2, 4, 5, 6, 7], 7: [1, 2, 3, 4, 5, 6, 7], 8: list(range(1, 9))}
    for b, rows in expect.items():
        np.testing.assert_array_equal(oracle.select_topb(ks, b)[0], rows)
        np.testing.assert_array_equal(_lexsort_top(ks[0], list(range(1, 9)), b), rows)


def test_topb_bos_never_a_candidate():
    ks = np.array([[1e30, 1.0, 2.0, 3.0]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.select_topb(ks, 1)[0], [3])
    np.testing.assert_array_equal(oracle.select_topb(ks, 3)[0], [1, 2, 3])


@pytest.mark.parametrize("seed", range(4))
def test_topk_matches_lexsort(seed):
    rng = np.random.default_rng(100 + seed)
    n_seq, n = 3, 40
    cs = rng.integers(0, 8, size=(n_seq, n)).astype(np.float32)
    kps = [0, 5, n] if seed == 0 else list(rng.integers(0, n + 1, size=n_seq))
    k_max = max(kps) + 2
    sel = oracle.select_topk(cs, kps, k_max)
    for s in range(n_seq):
        np.testing.assert_array_equal(sel[s, :kps[s]], _lexsort_top(cs[s], list(range(n)), kps[s]))
        assert np.all(sel[s, kps[s]:] == -1)


def test_topk_all_chunks_is_identity():
    cs = np.random.default_rng(0).random((2, 9)).astype(np.float32)
    sel = oracle.select_topk(cs, [9, 9], 9)
    np.testing.assert_array_equal(sel, np.tile(np.arange(9), (2, 1)))
