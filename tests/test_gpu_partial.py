"""GPU parity, through the C ABI, on prefixes that end in a partial chunk (a
chunk of C' < C tokens after its BOS, R_c = C' + 1 rows at the start of an
ordinary slot).  The slot and query rows past R_c hold large values, so any
use of them shows:

* chunk prefill with chunk_rows (on-chip bf16 kernel, streamed bf16 kernels
  for long chunks, float32 kernel) against the fp64 oracle over each chunk's
  own rows; keys past R_c must score exactly 0;
* top-B with chunk_rows, bit-exact, including the -1 padding of a chunk with
  fewer than B content rows;
* split decode with absent (-1) kept-row entries, at several split counts,
  including splits whose 64-row tiles are all absent;
* the chain prefill -> top-B -> top-K -> decode against the oracle's chain;
* compaction with absent entries, and the decode over those compacted slots.
"""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, max_abs, rel_l2, say

pytestmark = pytest.mark.gpu


def _prefill_gpu(inp, cfg):
    import torch
    from diffusion_long_context_amd import _lib as L
    o, ks = L.chunk_prefill_score(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(inp.q_chunk),
                                  dev(inp.q_win), cfg.n_chunks, cfg.scale, chunk_rows=dev(cfg.chunk_rows))
    torch.cuda.synchronize()
    return o, ks


def _check_prefill(o, ks, ro, rks, cfg, what):
    rows = cfg.chunk_rows
    valid = np.arange(cfg.rows)[None, :] < rows[:, None]             # [n_chunks][R]
    oh = host(o)
    assert_close(oh[valid], ro[valid], cfg.dtype, f"{what} o_chunk")
    ksh = host(ks)
    assert (ksh[~valid] == 0).all(), f"{what}: keys past R_c scored"
    r = rel_l2(ksh, rks)
    assert r <= TOL[cfg.dtype]["score_rel_l2"], f"{what}: key_score rel-L2 {r:.2e}"
    say(f"  {what}: key_score rel-L2 {r:.2e}")


PREFILL = [
    # (name, config); chunk 256 -> the on-chip kernel, 512 / 1024 -> streamed
    ("bf16_c256_last100", synth.Config("p", 28, 4, 128, "bf16", 3, 256, (2,), 128, 64, 64, n_seq=2, last_chunk=100)),
    ("bf16_c256_last1", synth.Config("p", 14, 2, 128, "bf16", 3, 256, (2,), 64, 32, 32, last_chunk=1)),
    ("bf16_c256_last250", synth.Config("p", 14, 2, 64, "bf16", 2, 256, (2,), 64, 40, 33, last_chunk=250)),
    ("bf16_c64_last30", synth.Config("p", 8, 2, 128, "bf16", 4, 64, (2,), 32, 20, 17, last_chunk=30)),
    ("bf16_c512_last300", synth.Config("p", 14, 2, 128, "bf16", 2, 512, (2,), 128, 64, 64, last_chunk=300)),
    ("bf16_c1024_last17", synth.Config("p", 8, 2, 64, "bf16", 2, 1024, (2,), 128, 48, 48, last_chunk=17)),
    # R_c = 129: a single row past the last 64-row tile of the partial chunk
    ("bf16_c512_last128", synth.Config("p", 14, 2, 128, "bf16", 2, 512, (2,), 128, 40, 40, last_chunk=128)),
    ("f32_c64_last20", synth.Config("p", 2, 1, 64, "f32", 4, 64, (2,), 16, 32, 32, last_chunk=20)),
]


@pytest.mark.parametrize("name,cfg", PREFILL, ids=[p[0] for p in PREFILL])
def test_partial_chunk_prefill(device, name, cfg):
    inp = synth.generate(cfg, 0, with_q_chunk=True)
    say(f"partial prefill {name}: oracle")
    ro, rks = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                         cfg.n_chunks, cfg.scale, chunk_rows=cfg.chunk_rows)
    say(f"partial prefill {name}: gpu")
    o, ks = _prefill_gpu(inp, cfg)
    _check_prefill(o, ks, ro, rks, cfg, name)


@pytest.mark.parametrize("b", [1, 40, 100, 101, 256])
def test_partial_chunk_topb(device, b):
    """Top-B over the GPU's own key scores, with chunk_rows: bit-exact."""
    from diffusion_long_context_amd import _lib as L
    cfg = synth.Config("p", 14, 2, 128, "bf16", 3, 256, (2,), b, 32, 32, n_seq=2, last_chunk=100)
    inp = synth.generate(cfg, 1, with_q_chunk=True)
    say(f"partial top-B b={b}")
    _, ks = _prefill_gpu(inp, cfg)
    keep = L.select_topb(ks, b, chunk_rows=dev(cfg.chunk_rows))
    want = oracle.select_topb(ks.cpu().numpy(), b, chunk_rows=cfg.chunk_rows)
    got = keep.cpu().numpy()
    assert np.array_equal(got, want)
    assert (got[cfg.chunk_rows < cfg.rows, 100:] == -1).all()


def _decode_gpu(inp, sel, keep, cfg, ns):
    import torch
    from diffusion_long_context_amd import _lib as L
    o, lse = L.split_attn_decode(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(sel), dev(keep),
                                 cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale,
                                 num_splits=ns)
    torch.cuda.synchronize()
    return host(o), host(lse)


DECODE = [
    # every chunk selected, so the partial one is attended; with B = 128 and
    # one token in the partial chunk, 127 consecutive absent rows hold a whole
    # 64-row tile
    ("bf16_d128_last1", synth.Config("d", 28, 4, 128, "bf16", 5, 256, (5,), 128, 32, 4, last_chunk=1)),
    ("bf16_d128_last60", synth.Config("d", 14, 2, 128, "bf16", 4, 256, (4, 2), 100, 40, 4, n_seq=2,
                                      last_chunk=60)),
    ("bf16_d64_last3", synth.Config("d", 8, 2, 64, "bf16", 4, 64, (4,), 40, 20, 4, last_chunk=3)),
    ("f32_d64_last1", synth.Config("d", 2, 1, 64, "f32", 4, 64, (4,), 40, 24, 4, last_chunk=1)),
]


@pytest.mark.parametrize("name,cfg", DECODE, ids=[d[0] for d in DECODE])
def test_decode_with_absent_rows(device, name, cfg):
    inp = synth.generate(cfg, 0)
    sel, keep = synth.random_page_table(cfg, 0)
    if cfg.k_per_seq[0] == cfg.n_chunks:
        sel[0, :] = np.arange(cfg.n_chunks)
    assert (keep == -1).any()
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                        inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    n_tiles = -(-(max(cfg.k_per_seq) * (cfg.b + 1) + cfg.l_d) // 64)
    for ns in (0, 1, 3, n_tiles):
        say(f"decode {name} num_splits={ns}")
        o, lse = _decode_gpu(inp, sel, keep, cfg, ns)
        r, m = assert_close(o, ro, cfg.dtype, f"{name} splits {ns}")
        ml = max_abs(lse, rlse)
        assert ml <= TOL[cfg.dtype]["lse"], f"{name} splits {ns}: lse {ml:.2e}"
        say(f"  rel-L2 {r:.2e} max-abs {m:.2e} lse {ml:.2e}")


def test_chain_with_partial_last_chunk(device):
    """prefill -> top-B -> top-K -> decode over a prefix with a partial last
    chunk, against the oracle's chain (top-B compared on the GPU's scores)."""
    import torch
    from diffusion_long_context_amd import _lib as L
    cfg = synth.Config("chain", 28, 4, 128, "bf16", 6, 256, (6, 3), 128, 64, 64, n_seq=2, last_chunk=77)
    inp = synth.generate(cfg, 2, with_q_chunk=True)
    rows_d = dev(cfg.chunk_rows)
    say("chain: gpu")
    _, ks = L.chunk_prefill_score(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(inp.q_chunk),
                                  dev(inp.q_win), cfg.n_chunks, cfg.scale, chunk_rows=rows_d)
    keep = L.select_topb(ks, cfg.b, chunk_rows=rows_d)
    sel = L.select_topk(dev(inp.chunk_score), cfg.k_per_seq, cfg.k_max)
    o, lse = L.split_attn_decode(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), sel, keep, cfg.k_per_seq,
                                 dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    torch.cuda.synchronize()
    keep_h, sel_h = keep.cpu().numpy(), sel.cpu().numpy()
    say("chain: oracle")
    assert np.array_equal(keep_h, oracle.select_topb(ks.cpu().numpy(), cfg.b, chunk_rows=cfg.chunk_rows))
    assert np.array_equal(sel_h, oracle.select_topk(inp.chunk_score, cfg.k_per_seq, cfg.k_max))
    assert (keep_h[cfg.chunk_rows < cfg.rows, 77:] == -1).all()
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel_h, keep_h, cfg.k_per_seq,
                                        inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    assert_close(host(o), ro, "bf16", "chain decode")
    assert max_abs(host(lse), rlse) <= TOL["bf16"]["lse"]


def test_compaction_with_absent_rows(device):
    import torch
    from diffusion_long_context_amd import _lib as L
    cfg = synth.Config("c", 28, 4, 128, "bf16", 5, 256, (5,), 128, 32, 4, last_chunk=9)
    inp = synth.generate(cfg, 3)
    sel, keep = synth.random_page_table(cfg, 3)
    sel[0, :] = np.arange(cfg.n_chunks)
    pk, pv, slot = dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot)
    say("compaction with absent rows")
    ck = torch.full((cfg.n_slots, cfg.b + 1, cfg.h_kv, cfg.d), 5.0, dtype=pk.dtype, device=pk.device)
    cv = torch.full_like(ck, 5.0)
    L.compact_kept_rows(pk, pv, slot, dev(keep), ck, cv)
    torch.cuda.synchronize()
    rk, rv, written = oracle.compact_kept_rows(inp.pool_k, inp.pool_v, inp.chunk_slot, keep, cfg.n_slots)
    bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits(ck)[written], rk[written]) and np.array_equal(bits(cv)[written], rv[written])
    assert (host(ck)[~written] == 5.0).all()                     # absent rows are not written
    rest = (cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    o_g, l_g = L.split_attn_decode(pk, pv, slot, dev(sel), dev(keep), *rest, num_splits=3)
    o_c, l_c = L.split_attn_decode(ck, cv, slot, dev(sel), dev(keep), *rest, num_splits=3, compacted=True)
    torch.cuda.synchronize()
    assert torch.equal(o_g, o_c) and torch.equal(l_g, l_c)
    ro, _ = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq, inp.q,
                                     inp.k_resp, inp.v_resp, cfg.scale)
    assert_close(host(o_c), ro, "bf16", "compacted decode with absent rows")
