"""Seeded random shapes through the whole path, GPU against the fp64 oracle:
chunk prefill with scoring, top-B over the GPU's own key scores, top-K, and
the decode (the planner's plan, a random forced split count, and the decode
without splits).  Each
case draws its sizes from its own seed: GQA group, head count, d, dtype,
chunk size (some past the 288 rows held on chip, so the streamed path runs,
and some multiples of 64, so one row is left past the last 64-row block),
partial last chunks, B from 0 to C, K_s from 0 to N per sequence, L_d and W,
and the key distribution.  Sizes stay small enough for the oracle to finish
in about a second per case."""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, max_abs, rel_l2, say

pytestmark = pytest.mark.gpu

N_CASES = 40


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    d = int(rng.choice([32, 64])) if dtype == "f32" else int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4, 7]))
    h_kv = int(rng.choice([1, 2]))
    n_seq = int(rng.integers(1, 4))
    n_chunks = int(rng.integers(1, 6))
    long = dtype == "bf16" and rng.random() < 0.2
    chunk = int(rng.integers(289, 420)) if long else int(rng.integers(1, 200))
    if rng.random() < 0.25:                  # C + 1 = 64 k + 1: the one-row tail
        chunk = int(rng.choice([64, 128, 192, 256, 320, 384] if dtype == "bf16" else [64, 128]))
    last = int(rng.integers(1, chunk + 1)) if rng.random() < 0.4 else 0
    b = int(rng.integers(0, chunk + 1))
    l_d = int(rng.integers(1, 90))
    w = int(rng.integers(1, l_d + 1))
    k_per_seq = tuple(int(rng.integers(0, n_chunks + 1)) for _ in range(n_seq))
    key_dist = "t4" if rng.random() < 0.3 else "normal"
    return synth.Config(f"fuzz{i}", g * h_kv, h_kv, d, dtype, n_chunks, chunk, k_per_seq, b, l_d, w,
                        n_seq=n_seq, key_dist=key_dist, key_offset_std=float(rng.choice([0.0, 0.5])),
                        last_chunk=last), int(rng.integers(1, 12))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shapes(device, i):
    import torch
    from diffusion_long_context_amd import _lib as L
    cfg, forced = _draw(i)
    say(f"fuzz {i}: {cfg}")
    inp = synth.generate(cfg, i, with_q_chunk=True)
    rows = cfg.chunk_rows
    rows_d = dev(rows) if cfg.last_chunk else None

    # chunk prefill and per-key scores
    o, ks = L.chunk_prefill_score(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(inp.q_chunk),
                                  dev(inp.q_win), cfg.n_chunks, cfg.scale, chunk_rows=rows_d)
    torch.cuda.synchronize()
    ro, rks = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                         cfg.n_chunks, cfg.scale, chunk_rows=rows if cfg.last_chunk else None)
    valid = np.arange(cfg.rows)[None, :] < rows[:, None]
    # rows past a partial chunk's R_c are not written (left as allocated)
    assert_close(host(o[torch.from_numpy(valid).to(o.device)]), ro[valid], cfg.dtype, f"fuzz {i} o_chunk")
    ksh = host(ks)
    r = rel_l2(ksh, rks)
    assert r <= TOL[cfg.dtype]["score_rel_l2"], f"fuzz {i}: key_score rel-L2 {r:.2e}"

    # selections: top-B over the GPU's scores, top-K over the given chunk scores
    keep = L.select_topb(ks, cfg.b, chunk_rows=rows_d)
    sel = L.select_topk(dev(inp.chunk_score), cfg.k_per_seq, cfg.k_max)
    torch.cuda.synchronize()
    keep_h, sel_h = keep.cpu().numpy(), sel.cpu().numpy()
    assert np.array_equal(keep_h, oracle.select_topb(ks.cpu().numpy(), cfg.b,
                                                     chunk_rows=rows if cfg.last_chunk else None))
    assert np.array_equal(sel_h, oracle.select_topk(inp.chunk_score, cfg.k_per_seq, cfg.k_max))

    # split decode over those selections
    rd, rl = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel_h, keep_h, cfg.k_per_seq,
                                      inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    # the planner's plan, a forced split count, and (bf16, pool rows within
    # its table) the decode without splits
    runs = [(0, 0), (forced, 0)]
    if cfg.dtype == "bf16" and max(cfg.k_per_seq) * (cfg.b + 1) <= 4864:
        runs.append((0, 32))
    for ns, qrows in runs:
        od, ld = L.split_attn_decode(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), sel, keep,
                                     cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale,
                                     num_splits=ns, q_rows_per_wg=qrows)
        torch.cuda.synchronize()
        assert_close(host(od), rd, cfg.dtype, f"fuzz {i} decode splits {ns} rows {qrows}")
        m = max_abs(host(ld), rl)
        assert m <= TOL[cfg.dtype]["lse"], f"fuzz {i} splits {ns} rows {qrows}: lse {m:.2e}"
    say(f"  fuzz {i} ok")
