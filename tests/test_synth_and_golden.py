"""Generator stability and the oracle's Tiny regression fixture."""
import json
import os

import numpy as np
import pytest

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bf16_rounding_is_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)                  # bf16 spacing at 1.0
    x = np.array([one + ulp / 2,                 # tie -> even (1.0)
                  one + 3 * ulp / 2,             # tie -> even (1 + 2 ulp)
                  one + ulp / 2 + np.float32(2.0 ** -20),   # above tie -> up
                  -(one + ulp / 2)], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    np.testing.assert_array_equal(bits, [0x3F80, 0x3F82, 0x3F81, 0xBF80])


def test_generator_is_deterministic_and_shaped():
    cfg = synth.config("tiny")
    a = synth.generate(cfg, 0, with_q_chunk=True)
    b = synth.generate(cfg, 0, with_q_chunk=True)
    assert a.sha256() == b.sha256()
    assert a.pool_k.shape == (8, 65, 1, 64) and a.pool_k.dtype == np.float32
    assert a.q_chunk.shape == (8, 65, 1, 64)
    assert sorted(a.chunk_slot.tolist()) == list(range(8))
    assert np.unique(a.chunk_score).size == a.chunk_score.size
    assert np.all((a.chunk_score >= 0) & (a.chunk_score < 1))
    c = synth.generate(cfg, 1)
    assert c.sha256()["pool_k"] != a.sha256()["pool_k"]


def test_bf16_config_shapes():
    cfg = synth.config("s8", n_chunks=4)
    a = synth.generate(cfg, 0)
    assert a.pool_k.dtype == np.uint16 and a.pool_k.shape == (4, 257, 4, 128)
    assert a.q.shape == (1, 256, 28, 128) and a.q_win.shape == (1, 64, 28, 128)


def test_random_page_table_is_valid():
    cfg = synth.config("s128", n_chunks=20, chunk=16, b=5, k_per_seq=(0, 3, 20, 7))
    sel, keep = synth.random_page_table(cfg, 0)
    assert sel.shape == (4, 20) and keep.shape == (80, 5)
    for s, ks in enumerate(cfg.k_per_seq):
        row = sel[s]
        assert np.all(np.diff(row[:ks]) > 0) and np.all(row[ks:] == -1)
        assert np.all((row[:ks] >= 0) & (row[:ks] < 20))
    assert np.all(np.diff(keep, axis=1) > 0) and keep.min() >= 1 and keep.max() <= 16


def test_tiny_golden_regression():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    got = mg.summary(mg.tiny_chain(0))
    with open(os.path.join(HERE, "golden", "tiny_seed0.json")) as f:
        want = json.load(f)
    assert got["sel_chunk"] == want["sel_chunk"]
    assert got["keep_rows"] == want["keep_rows"]
    for key in ("key_score_sum", "o_chunk_sum", "o_chunk_sumsq", "o_sum", "o_sumsq"):
        assert got[key] == pytest.approx(want[key], rel=1e-12, abs=1e-12)
    for key in ("key_score_first_chunk", "o_row0", "lse"):
        np.testing.assert_allclose(got[key], want[key], rtol=1e-12, atol=1e-12)
