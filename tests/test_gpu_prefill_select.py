"""GPU parity of pdllm_prefill_select (chunk prefill, key-score finalize,
top-B and top-K in one call) through the C ABI: its outputs equal those of
pdllm_chunk_prefill_score + pdllm_select_topB + pdllm_select_topK bit for
bit, and its selections equal the oracle's on the same score arrays.  Covers
the 32K workload, several sequences (more than one top-K launch's worth too),
a partial last chunk, streamed chunks, float32, B = 0 and K = 0."""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, rel_l2, say

pytestmark = pytest.mark.gpu


def _both(cfg, seed, b=None, k_max=None, chunk_rows=None):
    import torch
    from diffusion_long_context_amd import _lib as L
    b = cfg.b if b is None else b
    k_per_seq = list(cfg.k_per_seq) if k_max is None else [min(k, k_max) for k in cfg.k_per_seq]
    k_max = cfg.k_max if k_max is None else k_max
    inp = synth.generate(cfg, seed, with_q_chunk=True)
    pk, pv, slot = dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot)
    qc, qw, cs = dev(inp.q_chunk), dev(inp.q_win), dev(inp.chunk_score)
    rows = dev(chunk_rows) if chunk_rows is not None else None
    o1, ks1 = L.chunk_prefill_score(pk, pv, slot, qc, qw, cfg.n_chunks, cfg.scale, chunk_rows=rows)
    keep1 = L.select_topb(ks1, b, chunk_rows=rows)
    sel1 = L.select_topk(cs, k_per_seq, k_max)
    o2, ks2, keep2, sel2 = L.prefill_select(pk, pv, slot, qc, qw, cfg.n_chunks, cfg.scale, b, cs, k_per_seq, k_max,
                                            chunk_rows=rows)
    torch.cuda.synchronize()
    return inp, (o1, ks1, keep1, sel1), (o2, ks2, keep2, sel2), b, k_per_seq, k_max


def _check(cfg, sep, fused, inp, b, k_per_seq, k_max, chunk_rows=None, what=""):
    import torch
    o1, ks1, keep1, sel1 = sep
    o2, ks2, keep2, sel2 = fused
    rows = cfg.chunk_rows if chunk_rows is None else chunk_rows
    valid = torch.from_numpy(np.arange(cfg.rows)[None, :] < rows[:, None]).to(o1.device)
    assert torch.equal(o1[valid], o2[valid]), f"{what}: o_chunk differs"
    assert torch.equal(ks1, ks2), f"{what}: key_score differs"
    assert torch.equal(keep1, keep2), f"{what}: keep_rows differs"
    assert torch.equal(sel1, sel2), f"{what}: sel_chunk differs"
    ks = ks2.cpu().numpy()
    assert np.array_equal(keep2.cpu().numpy(), oracle.select_topb(ks, b, chunk_rows=chunk_rows))
    if k_max:
        assert np.array_equal(sel2.cpu().numpy(), oracle.select_topk(inp.chunk_score, k_per_seq, k_max))


CASES = [
    ("s32", synth.config("s32"), {}),
    ("two_seq", synth.Config("p", 28, 4, 128, "bf16", 6, 256, (3, 5), 100, 64, 64, n_seq=2), {}),
    ("b0", synth.Config("p", 14, 2, 128, "bf16", 4, 64, (2,), 0, 32, 32), {}),
    ("k0", synth.Config("p", 14, 2, 64, "bf16", 4, 64, (2,), 20, 32, 32), dict(k_max=0)),
    ("c512", synth.Config("p", 14, 2, 128, "bf16", 3, 512, (2,), 200, 64, 64), {}),
    ("tiny_f32", synth.config("tiny"), {}),
]


@pytest.mark.parametrize("name,cfg,kw", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_separate_calls(device, name, cfg, kw):
    say(f"prefill_select {name}")
    inp, sep, fused, b, ks, k_max = _both(cfg, 0, **kw)
    _check(cfg, sep, fused, inp, b, ks, k_max, what=name)


def test_fused_with_partial_last_chunk(device):
    cfg = synth.Config("p", 28, 4, 128, "bf16", 4, 256, (4, 2), 128, 64, 64, n_seq=2, last_chunk=60)
    say("prefill_select, partial last chunk")
    inp, sep, fused, b, ks, k_max = _both(cfg, 1, chunk_rows=cfg.chunk_rows)
    _check(cfg, sep, fused, inp, b, ks, k_max, chunk_rows=cfg.chunk_rows, what="partial")
    assert (fused[2].cpu().numpy()[cfg.chunk_rows < cfg.rows, 60:] == -1).all()


def test_fused_with_many_sequences(device):
    """70 sequences: top-K needs a second launch past the fused one."""
    cfg = synth.Config("p", 4, 2, 64, "bf16", 3, 32, tuple([1, 2, 3, 0] * 17 + [2, 1]), 8, 16, 16, n_seq=70)
    say("prefill_select, 70 sequences")
    inp, sep, fused, b, ks, k_max = _both(cfg, 2)
    _check(cfg, sep, fused, inp, b, ks, k_max, what="70 sequences")


SELECTED = [
    ("s32", synth.config("s32"), None),
    ("two_seq_partial", synth.Config("p", 28, 4, 128, "bf16", 6, 256, (3, 5), 100, 64, 64, n_seq=2, last_chunk=50),
     "rows"),
    ("k0", synth.Config("p", 14, 2, 64, "bf16", 4, 64, (0,), 20, 32, 32), None),
    ("c512", synth.Config("p", 14, 2, 128, "bf16", 4, 512, (2,), 200, 64, 64), None),
    ("tiny_f32", synth.config("tiny"), None),
    ("70_seq", synth.Config("p", 4, 2, 64, "bf16", 3, 32, tuple([1, 2, 3, 0] * 17 + [2, 1]), 8, 16, 16, n_seq=70),
     None),
]


@pytest.mark.parametrize("name,cfg,rows_kind", SELECTED, ids=[c[0] for c in SELECTED])
def test_selected_only(device, name, cfg, rows_kind):
    """selected_only: the chunks top-K selects get the key scores and kept rows
    of the full call bit for bit; the others' rows are not written (past 64
    sequences every chunk is); o_chunk and sel_chunk equal the full call's."""
    import torch
    from diffusion_long_context_amd import _lib as L
    inp = synth.generate(cfg, 3, with_q_chunk=True)
    rows = dev(cfg.chunk_rows) if rows_kind else None
    pk, pv, slot = dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot)
    qc, qw, cs = dev(inp.q_chunk), dev(inp.q_win), dev(inp.chunk_score)
    say(f"selected_only {name}")
    full = L.prefill_select(pk, pv, slot, qc, qw, cfg.n_chunks, cfg.scale, cfg.b, cs, cfg.k_per_seq, cfg.k_max,
                            chunk_rows=rows)
    ks_m = torch.full((cfg.n_slots, cfg.rows), -7.0, dtype=torch.float32, device=qc.device)
    keep_m = torch.full((cfg.n_slots, cfg.b), -9, dtype=torch.int32, device=qc.device)
    part = L.prefill_select(pk, pv, slot, qc, qw, cfg.n_chunks, cfg.scale, cfg.b, cs, cfg.k_per_seq, cfg.k_max,
                            chunk_rows=rows, key_score=ks_m, keep_rows=keep_m, selected_only=True)
    torch.cuda.synchronize()
    sel = oracle.select_topk(inp.chunk_score, cfg.k_per_seq, cfg.k_max)
    picked = np.zeros(cfg.n_slots, dtype=bool)
    for s in range(cfg.n_seq):
        for c in sel[s, :cfg.k_per_seq[s]]:
            picked[s * cfg.n_chunks + c] = True
    if cfg.n_seq > 64:
        picked[:] = True                    # past 64 sequences every chunk is scored
    pk_t = torch.from_numpy(picked).to(qc.device)
    valid = np.arange(cfg.rows)[None, :] < cfg.chunk_rows[:, None]
    valid_t = torch.from_numpy(valid).to(qc.device)
    assert torch.equal(full[0][valid_t], part[0][valid_t]), "o_chunk"
    assert torch.equal(full[1][pk_t], part[1][pk_t]), "key_score of selected chunks"
    assert torch.equal(full[2][pk_t], part[2][pk_t]), "keep_rows of selected chunks"
    assert torch.equal(full[3], part[3]), "sel_chunk"
    assert (part[1][~pk_t] == -7.0).all() and (part[2][~pk_t] == -9).all(), "unselected chunks were written"
    assert picked.any() or cfg.k_max == 0


def _e2e_selection(cfg, chunks, ks_gpu, keep_gpu, rks, what):
    """End-to-end selection: the GPU's top-B rows (from its float32 key
    scores) against the oracle's top-B from its float64 scores, exact at
    every chunk whose fp64 cut gap |s_(B) - s_(B+1)| exceeds four times that
    chunk's largest score error; near-tie chunks are reported, not failed."""
    near = []
    for n, c in enumerate(chunks):
        err = float(np.abs(ks_gpu[c].astype(np.float64) - rks[n]).max())
        ref = oracle.select_topb(rks[n:n + 1], cfg.b)[0]
        srt = np.sort(rks[n, 1:])[::-1]
        gap = srt[cfg.b - 1] - srt[cfg.b] if cfg.b < cfg.chunk else np.inf
        if gap > 4 * err:
            assert np.array_equal(keep_gpu[c], ref), f"{what}: chunk {c} selection differs from the fp64 oracle's"
        else:
            near.append((c, gap, err))
    say(f"  {what}: {len(chunks)} chunks checked end to end, near ties: {near}")


SEL_E2E = [("s32", synth.config("s32"), 0), ("s8", synth.config("s8"), 0), ("f32", synth.config("f32"), 0)]


@pytest.mark.parametrize("name,cfg,seed", SEL_E2E, ids=[c[0] for c in SEL_E2E])
def test_selected_only_against_oracle(device, name, cfg, seed):
    """The benched form of the prefill side, pdllm_prefill_select with
    selected_only, compared with the oracle directly: o_chunk on sampled
    chunks (kept and not kept), the key scores of every kept chunk, top-K,
    top-B on the GPU's own scores (bit-exact) and against the fp64 scores
    (end to end, exact outside near ties).  S8 and F32 keep B = 128 < C."""
    import torch
    from diffusion_long_context_amd import _lib as L
    say(f"selected_only vs oracle {name}: generating")
    inp = synth.generate(cfg, seed, with_q_chunk=True)
    pk, pv, slot = dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot)
    qc, qw, cs = dev(inp.q_chunk), dev(inp.q_win), dev(inp.chunk_score)
    say(f"selected_only vs oracle {name}: gpu")
    o, ks, keep, sel = L.prefill_select(pk, pv, slot, qc, qw, cfg.n_chunks, cfg.scale, cfg.b, cs, cfg.k_per_seq,
                                        cfg.k_max, selected_only=True)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    assert np.array_equal(sel_h, oracle.select_topk(inp.chunk_score, cfg.k_per_seq, cfg.k_max)), "top-K"
    kept = sorted(int(c) for c in sel_h[0, :cfg.k_per_seq[0]])
    say(f"selected_only vs oracle {name}: oracle on the {len(kept)} kept chunks")
    ro, rks = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                         cfg.n_chunks, cfg.scale, chunks=kept)
    ks_h, keep_h, o_h = ks.cpu().numpy(), keep.cpu().numpy(), host(o)
    r = rel_l2(ks_h[kept], rks)
    assert r <= TOL["bf16"]["score_rel_l2"], f"{name}: key_score rel-L2 {r:.2e}"
    assert_close(o_h[kept], ro, "bf16", f"{name}: o_chunk of kept chunks")
    assert np.array_equal(keep_h[kept], oracle.select_topb(ks_h[kept], cfg.b)), "top-B on the GPU's scores"
    _e2e_selection(cfg, kept, ks_h, keep_h, rks, f"{name} selected_only")
    others = [c for c in (0, cfg.n_chunks // 2, cfg.n_chunks - 1) if c not in kept][:2]
    ro2, _ = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                        cfg.n_chunks, cfg.scale, chunks=others)
    assert_close(o_h[others], ro2, "bf16", f"{name}: o_chunk of chunks not kept")


def test_all_chunks_scored_end_to_end_s8(device):
    """Every chunk scored (selected_only = 0) at S8: all 32 chunks' top-B
    rows against the fp64 oracle's, end to end."""
    import torch
    from diffusion_long_context_amd import _lib as L
    cfg = synth.config("s8")
    inp = synth.generate(cfg, 1, with_q_chunk=True)
    _, ks, keep, _ = L.prefill_select(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(inp.q_chunk),
                                      dev(inp.q_win), cfg.n_chunks, cfg.scale, cfg.b, dev(inp.chunk_score),
                                      cfg.k_per_seq, cfg.k_max)
    torch.cuda.synchronize()
    say("s8 all chunks: oracle")
    _, rks = oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                                        cfg.n_chunks, cfg.scale)
    ks_h, keep_h = ks.cpu().numpy(), keep.cpu().numpy()
    assert rel_l2(ks_h, rks) <= TOL["bf16"]["score_rel_l2"]
    _e2e_selection(cfg, list(range(cfg.n_slots)), ks_h, keep_h, rks, "s8 all chunks")
