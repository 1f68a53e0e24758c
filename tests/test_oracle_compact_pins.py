"""Pins of the oracle's kept-row compaction (Prefilling-dLLM summary,
Methodology 2: after the intra-chunk selection only a chunk's top-B tokens
stay in the KV cache, with its BOS anchor), independent of the oracle's own
indexing:

* every pool value encodes its own (slot, row, head), so each compacted row
  can be checked against the coordinates it must come from, computed from
  the encoding rather than by indexing the pool;
* B = C keeps every row, so the compacted slots equal the pool's;
* decode attention over the compacted slots with rows 1..B equals decode
  attention over the whole-chunk pool with the keep_rows table: the two
  attended sets are the same rows in the same order.
"""
import numpy as np
import pytest

import oracle
import synth


def _encoded_pool(n_slots, rows, h_kv, d):
    """K[s, r, h, :] = 100000 s + 100 r + h and V = -K (exact in float32)."""
    s = np.arange(n_slots)[:, None, None, None]
    r = np.arange(rows)[None, :, None, None]
    h = np.arange(h_kv)[None, None, :, None]
    k = np.broadcast_to(100000.0 * s + 100.0 * r + h, (n_slots, rows, h_kv, d)).astype(np.float32)
    return k, -k


def _random_keep(rng, n_chunks, c, b):
    return np.stack([np.sort(rng.choice(np.arange(1, c + 1), size=b, replace=False))
                     for _ in range(n_chunks)]).astype(np.int32)


@pytest.mark.parametrize("b", [0, 1, 5, 12])
def test_compacted_rows_carry_their_source_coordinates(b):
    rng = np.random.default_rng(7 + b)
    n_slots, c, h_kv, d = 9, 12, 3, 4
    pk, pv = _encoded_pool(n_slots, c + 1, h_kv, d)
    chunk_slot = rng.permutation(n_slots).astype(np.int32)
    n_chunks = 7                                   # two slots hold no listed chunk
    keep = _random_keep(rng, n_chunks, c, b)
    k, v, written = oracle.compact_kept_rows(pk, pv, chunk_slot, keep, n_chunks)
    assert k.shape == (n_slots, b + 1, h_kv, d) and k.dtype == np.float32
    for ch in range(n_chunks):
        slot = int(chunk_slot[ch])
        src_rows = [0] + list(keep[ch])
        for j, r in enumerate(src_rows):
            for h in range(h_kv):
                want = 100000.0 * slot + 100.0 * r + h
                assert np.all(k[slot, j, h] == want), (ch, j, h)
                assert np.all(v[slot, j, h] == -want), (ch, j, h)
    listed = set(int(x) for x in chunk_slot[:n_chunks])
    assert set(np.flatnonzero(written.any(axis=1))) == listed and written[sorted(listed)].all()
    for slot in set(range(n_slots)) - listed:
        assert not k[slot].any() and not v[slot].any()


def test_keeping_every_row_copies_the_slots():
    cfg = synth.Config("pin", 4, 2, 8, "bf16", 6, 10, (3,), 10, 4, 4)
    inp = synth.generate(cfg, 3)
    keep = oracle.all_rows_kept(cfg.n_chunks, cfg.chunk)
    k, v, written = oracle.compact_kept_rows(inp.pool_k, inp.pool_v, inp.chunk_slot, keep, cfg.n_chunks)
    assert written.all()
    assert k.dtype == np.uint16
    assert np.array_equal(k, inp.pool_k) and np.array_equal(v, inp.pool_v)


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_over_compacted_slots_equals_decode_with_keep_rows(seed):
    cfg = synth.Config("pin", 4, 2, 8, "f32", 6, 10, (4, 2), 5, 3, 3, n_seq=2)
    inp = synth.generate(cfg, seed)
    rng = np.random.default_rng(100 + seed)
    keep = _random_keep(rng, cfg.n_seq * cfg.n_chunks, cfg.chunk, cfg.b)
    sel = oracle.select_topk(inp.chunk_score, cfg.k_per_seq, cfg.k_max)
    o_ref, lse_ref = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep,
                                              cfg.k_per_seq, inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    k, v, _ = oracle.compact_kept_rows(inp.pool_k, inp.pool_v, inp.chunk_slot, keep,
                                       cfg.n_seq * cfg.n_chunks)
    ident = oracle.all_rows_kept(cfg.n_seq * cfg.n_chunks, cfg.b)
    o, lse = oracle.split_attn_decode(k, v, inp.chunk_slot, sel, ident, cfg.k_per_seq, inp.q,
                                      inp.k_resp, inp.v_resp, cfg.scale)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)


def test_all_rows_kept_lists_rows_one_to_b():
    t = oracle.all_rows_kept(3, 4)
    assert t.dtype == np.int32 and t.shape == (3, 4)
    assert (t == np.array([1, 2, 3, 4])).all()
    assert oracle.all_rows_kept(2, 0).shape == (2, 0)
