"""GPU parity of pdllm_chunk_prefill_score (chunk-local attention + per-key
window scores) against the fp64 oracle, and of the whole chain
prefill -> top-B -> top-K -> decode."""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu


def _prefill_gpu(inp, cfg, chunks_per_win=None):
    from diffusion_long_context_amd import _lib as L
    import torch
    cpw = cfg.n_chunks if chunks_per_win is None else chunks_per_win
    o, ks = L.chunk_prefill_score(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot),
                                  dev(inp.q_chunk), dev(inp.q_win), cpw, cfg.scale)
    torch.cuda.synchronize()
    return o, ks


def _check_prefill(inp, cfg, chunks=None, what=""):
    o, ks = _prefill_gpu(inp, cfg)
    ro, rks = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                         cfg.n_chunks, cfg.scale, chunks=chunks)
    idx = slice(None) if chunks is None else list(chunks)
    og, kg = host(o)[idx], host(ks)[idx]
    r, m = assert_close(og, ro, cfg.dtype, f"{what} o_chunk")
    rs = rel_l2(kg, rks)
    assert rs <= TOL[cfg.dtype]["score_rel_l2"], f"{what} key_score rel-L2 {rs:.3e}"
    # each chunk's scores add up to W * h_q (every window row's softmax sums to one)
    tot = host(ks).sum(axis=1)
    assert np.allclose(tot, cfg.w * cfg.h_q, rtol=1e-5, atol=0), f"{what} score sums {tot[:4]}"
    say(f"  {what}: o rel-L2 {r:.2e} max-abs {m:.2e}; score rel-L2 {rs:.2e}")
    return o, ks


def test_tiny_f32(device):
    cfg = synth.config("tiny")
    inp = synth.generate(cfg, 0, with_q_chunk=True)
    say("tiny prefill f32")
    _check_prefill(inp, cfg, what="tiny")


SMALL = [
    ("g7_c64", dict(h_q=7, h_kv=1, d=128, n_chunks=5, chunk=64, w=16)),
    ("g7x4_c256", dict(h_q=28, h_kv=4, d=128, n_chunks=3, chunk=256, w=64)),
    ("g2_d64_c33", dict(h_q=4, h_kv=2, d=64, n_chunks=4, chunk=33, w=5, n_seq=2)),
    ("g1_c8", dict(h_q=2, h_kv=2, d=128, n_chunks=6, chunk=8, w=3)),
    ("c100_w70", dict(h_q=7, h_kv=1, d=128, n_chunks=2, chunk=100, w=70)),
    ("f32_d32", dict(h_q=6, h_kv=3, d=32, dtype="f32", n_chunks=3, chunk=50, w=7)),
    # one row past the last 64-row block (the one-row update), at d = 64
    ("d64_c128_one_row", dict(h_q=4, h_kv=1, d=64, n_chunks=3, chunk=128, w=20)),
    # 27 rows past the last 64-row block (a masked 32-row step)
    ("c90_tail27", dict(h_q=7, h_kv=1, d=128, n_chunks=2, chunk=90, w=33)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes(device, name, kw):
    base = dict(name=name, dtype="bf16", k_per_seq=(1,), b=1, l_d=max(kw.get("w", 4), 4), n_seq=1)
    base.update(kw)
    cfg = synth.Config(**base)
    inp = synth.generate(cfg, 7, with_q_chunk=True)
    say(f"prefill {name}")
    _check_prefill(inp, cfg, what=name)


# Chunks longer than the 288 rows the one-pass kernel holds on chip stream
# their K and V instead: one row past that limit, the chunk sizes of the
# method's trade-off study (512 .. 4096), d = 64, window row counts that are
# not a multiple of 32, and a single window row.
STREAMED = [
    ("c288", dict(h_q=7, h_kv=1, d=128, n_chunks=2, chunk=288, w=64)),
    ("c512_g2", dict(h_q=4, h_kv=2, d=128, n_chunks=3, chunk=512, w=16)),
    ("c1024_g7", dict(h_q=7, h_kv=1, d=128, n_chunks=2, chunk=1024, w=64)),
    ("c2048_d64", dict(h_q=4, h_kv=2, d=64, n_chunks=2, chunk=2048, w=9)),
    ("c4096", dict(h_q=2, h_kv=1, d=128, n_chunks=2, chunk=4096, w=40)),
    ("c700_w1", dict(h_q=3, h_kv=3, d=128, n_chunks=2, chunk=700, w=1)),
]


@pytest.mark.parametrize("name,kw", STREAMED, ids=[s[0] for s in STREAMED])
def test_streamed_chunks(device, name, kw):
    base = dict(name=name, dtype="bf16", k_per_seq=(1,), b=1, l_d=max(kw.get("w", 4), 4), n_seq=1)
    base.update(kw)
    cfg = synth.Config(**base)
    inp = synth.generate(cfg, 11, with_q_chunk=True)
    say(f"streamed prefill {name} (slot rows {cfg.rows})")
    o, ks = _check_prefill(inp, cfg, what=name)
    o2, ks2 = _prefill_gpu(inp, cfg)
    assert np.array_equal(host(o), host(o2)) and np.array_equal(host(ks), host(ks2)), "not reproducible"


def test_streamed_identical_keys(device):
    """All keys equal: every window weight is 1/R, so every score is W h_q / R,
    and every chunk row's output is the mean of the slot's V rows."""
    cfg = synth.Config("same_long", 7, 1, 128, "bf16", 2, 600, (1,), 1, 24, 24)
    inp = synth.generate(cfg, 2, with_q_chunk=True)
    inp.pool_k[:] = inp.pool_k[0, 0]
    o, ks = _prefill_gpu(inp, cfg)
    assert np.allclose(host(ks), cfg.w * cfg.h_q / cfg.rows, rtol=1e-5, atol=0)
    vmean = oracle.as_f64(inp.pool_v).mean(axis=1)            # [n_slots][h_kv][d]
    og = host(o).astype(np.float64)
    for c in range(cfg.n_chunks):
        want = vmean[inp.chunk_slot[c], 0]
        assert np.abs(og[c] - want).max() <= 2e-2, f"chunk {c}"


def test_s32_sampled_chunks(device):
    cfg = synth.config("s32")
    say("s32 prefill: generating")
    inp = synth.generate(cfg, 0, with_q_chunk=True)
    chunks = [0, 1, 63, 64, 127]
    say("s32 prefill: gpu + oracle on sampled chunks")
    o, ks = _check_prefill(inp, cfg, chunks=chunks, what="s32")
    o2, ks2 = _prefill_gpu(inp, cfg)
    assert np.array_equal(host(o), host(o2)) and np.array_equal(host(ks), host(ks2)), "not reproducible"


def test_identical_keys_uniform_scores(device):
    cfg = synth.Config("same", 14, 2, 128, "bf16", 3, 40, (1,), 1, 8, 8)
    inp = synth.generate(cfg, 1, with_q_chunk=True)
    inp.pool_k[:] = inp.pool_k[0, 0]
    o, ks = _prefill_gpu(inp, cfg)
    assert np.allclose(host(ks), cfg.w * cfg.h_q / cfg.rows, rtol=1e-5, atol=0)


@pytest.mark.parametrize("name", ["tiny", "s8"])
def test_chain(device, name):
    """prefill -> top-B -> top-K -> decode on the GPU, each stage checked
    against the oracle on the same inputs the GPU stage received."""
    from diffusion_long_context_amd import _lib as L
    import torch
    cfg = synth.config(name)
    if name == "s8":
        cfg = synth.config("s8", n_chunks=32)
    inp = synth.generate(cfg, 0, with_q_chunk=True)
    say(f"chain {name}: prefill")
    o_chunk, ks = _prefill_gpu(inp, cfg)
    ro, rks = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                         cfg.n_chunks, cfg.scale, chunks=[0, 1])
    assert_close(host(o_chunk)[:2], ro, cfg.dtype, "chain o_chunk")
    say(f"chain {name}: top-B on the GPU's key scores")
    keep = L.select_topb(ks, cfg.b)
    ks_h = ks.cpu().numpy()
    keep_h = keep.cpu().numpy()
    assert np.array_equal(keep_h, oracle.select_topb(ks_h, cfg.b))
    # against the fp64 scores: exact wherever the cut is not a near-tie
    full_ro, full_rks = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk,
                                                   inp.q_win, cfg.n_chunks, cfg.scale) \
        if name == "tiny" else (None, None)
    if full_rks is not None:
        ref_keep = oracle.select_topb(full_rks, cfg.b)
        err = np.abs(ks_h - full_rks).max(axis=1)
        for c in range(cfg.n_slots):
            srt = np.sort(full_rks[c, 1:])[::-1]
            gap = srt[cfg.b - 1] - srt[cfg.b] if cfg.b < cfg.chunk else np.inf
            if gap > 4 * err[c]:
                assert np.array_equal(keep_h[c], ref_keep[c]), f"chunk {c}"
    say(f"chain {name}: top-K")
    sel = L.select_topk(dev(inp.chunk_score), cfg.k_per_seq, cfg.k_max)
    sel_h = sel.cpu().numpy()
    assert np.array_equal(sel_h, oracle.select_topk(inp.chunk_score, cfg.k_per_seq, cfg.k_max))
    say(f"chain {name}: decode over the GPU-selected page table")
    o, lse = L.split_attn_decode(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), sel, keep,
                                 cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    torch.cuda.synchronize()
    rdo, rdl = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel_h, keep_h,
                                        cfg.k_per_seq, inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    assert_close(host(o), rdo, cfg.dtype, "chain decode")
