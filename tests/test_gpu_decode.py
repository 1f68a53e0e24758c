"""GPU parity of pdllm_split_attn_decode against the fp64 oracle, through the
C ABI, on seeded inputs: the Tiny fp32 case, small bf16 shapes spanning
several tiles with ragged tails, the 8K / 32K / 128K workloads, forced split
counts, and the degenerate cases (no chunks, no kept rows, one row)."""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, max_abs, say

pytestmark = pytest.mark.gpu


def _run_gpu(inp, sel, keep, cfg, num_splits=0):
    from diffusion_long_context_amd import _lib as L
    call = L.Decode(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(sel), dev(keep),
                    cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale,
                    num_splits=num_splits)
    o, lse = call()
    import torch
    torch.cuda.synchronize()
    return host(o), host(lse)


def _oracle(inp, sel, keep, cfg, heads=None):
    return oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                    inp.q, inp.k_resp, inp.v_resp, cfg.scale, heads=heads)


def _compare(o, lse, ro, rlse, cfg, what, heads=None):
    kind = cfg.dtype
    if heads is not None:
        o, ro = o[:, :, heads], ro[:, :, heads]
        lse, rlse = lse[:, heads], rlse[:, heads]
    r, m = assert_close(o, ro, kind, what)
    ml = max_abs(lse, rlse)
    assert ml <= TOL[kind]["lse"], f"{what}: lse max-abs {ml:.3e}"
    say(f"  {what}: rel-L2 {r:.2e} max-abs {m:.2e} lse {ml:.2e}")


def test_tiny_f32(device):
    cfg = synth.config("tiny")
    inp = synth.generate(cfg, 0)
    sel, keep = synth.random_page_table(cfg, 0)
    ro, rlse = _oracle(inp, sel, keep, cfg)
    for ns in (0, 1, 2, 3):
        say(f"tiny f32 decode, num_splits={ns}")
        o, lse = _run_gpu(inp, sel, keep, cfg, ns)
        _compare(o, lse, ro, rlse, cfg, f"tiny splits={ns}")


SMALL = [
    # (name, overrides)
    ("g7_d128", dict(h_q=7, h_kv=1, d=128, n_chunks=6, chunk=40, k_per_seq=(3,), b=17, l_d=33)),
    ("g7x4_d128", dict(h_q=28, h_kv=4, d=128, n_chunks=5, chunk=64, k_per_seq=(2,), b=64, l_d=20)),
    ("g2_d64_multi", dict(h_q=4, h_kv=2, d=64, n_chunks=4, chunk=31, k_per_seq=(4, 0, 1), b=9, l_d=70,
                          n_seq=3)),
    ("g1_d64_b0", dict(h_q=3, h_kv=3, d=64, n_chunks=7, chunk=16, k_per_seq=(5,), b=0, l_d=5)),
    ("one_row", dict(h_q=8, h_kv=2, d=128, n_chunks=3, chunk=8, k_per_seq=(0,), b=2, l_d=1)),
    ("f32_d32", dict(h_q=6, h_kv=2, d=32, dtype="f32", n_chunks=5, chunk=20, k_per_seq=(3, 5), b=11,
                     l_d=9, n_seq=2)),
    ("f32_d128", dict(h_q=2, h_kv=1, d=128, dtype="f32", n_chunks=4, chunk=70, k_per_seq=(4,), b=70,
                      l_d=17)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes(device, name, kw):
    base = dict(name=name, dtype="bf16", w=4, n_seq=1)
    base.update(kw)
    cfg = synth.Config(**base)
    for seed in (0, 1):
        inp = synth.generate(cfg, seed)
        sel, keep = synth.random_page_table(cfg, seed)
        ro, rlse = _oracle(inp, sel, keep, cfg)
        for ns in (0, 1, 2, 5):
            say(f"{name} seed={seed} num_splits={ns}")
            o, lse = _run_gpu(inp, sel, keep, cfg, ns)
            _compare(o, lse, ro, rlse, cfg, f"{name} seed {seed} splits {ns}")


@pytest.mark.parametrize("name", ["s8", "s32", "f32"])
def test_full_size_single_sequence(device, name):
    cfg = synth.config(name)
    inp = synth.generate(cfg, 0)
    sel, keep = synth.random_page_table(cfg, 0)
    say(f"{name}: oracle")
    ro, rlse = _oracle(inp, sel, keep, cfg)
    say(f"{name}: gpu, planner's split count")
    o, lse = _run_gpu(inp, sel, keep, cfg, 0)
    _compare(o, lse, ro, rlse, cfg, f"{name} planner")


def test_s32_split_invariance(device):
    """Any forced split count gives the oracle's result (and nearly the same
    bits as one split)."""
    cfg = synth.config("s32")
    inp = synth.generate(cfg, 1)
    sel, keep = synth.random_page_table(cfg, 1)
    heads = [0, 6, 7, 13, 27]
    ro, rlse = _oracle(inp, sel, keep, cfg, heads=heads)
    base = None
    for ns in (1, 2, 3, 7, 23, 69):
        say(f"s32 num_splits={ns}")
        o, lse = _run_gpu(inp, sel, keep, cfg, ns)
        _compare(o, lse, ro, rlse, cfg, f"s32 splits {ns}", heads=heads)
        if base is None:
            base = o
        else:
            assert max_abs(o, base) <= 2 * 2 ** -8 * max(1.0, np.abs(base).max())


def test_s128_batch_sampled_heads(device):
    cfg = synth.config("s128")
    say("s128: generating inputs")
    inp = synth.generate(cfg, 0)
    sel, keep = synth.random_page_table(cfg, 0)
    heads = [0, 5, 9, 20, 27]
    say("s128: oracle on sampled heads")
    ro, rlse = _oracle(inp, sel, keep, cfg, heads=heads)
    say("s128: gpu")
    o, lse = _run_gpu(inp, sel, keep, cfg, 0)
    _compare(o, lse, ro, rlse, cfg, "s128", heads=heads)


def test_identical_keys_give_mean_of_values(device):
    cfg = synth.Config("same", 14, 2, 128, "bf16", 4, 48, (3,), 20, 40, 4)
    inp = synth.generate(cfg, 3)
    sel, keep = synth.random_page_table(cfg, 3)
    inp.pool_k[:] = inp.pool_k[0, 0]
    inp.k_resp[:] = inp.pool_k[0, 0]
    say("identical keys")
    o, _ = _run_gpu(inp, sel, keep, cfg, 2)
    ro, _ = _oracle(inp, sel, keep, cfg)
    _, vv = oracle.attended_kv(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, 3, 0, 4, inp.k_resp,
                               inp.v_resp)
    g_of = np.arange(cfg.h_q) // (cfg.h_q // cfg.h_kv)
    mean = vv.mean(axis=0)[g_of]                       # [h_q][d]
    assert_close(o[0], np.broadcast_to(mean, o[0].shape), "bf16", "identical keys")
    assert_close(o, ro, "bf16", "identical keys vs oracle")


def test_full_selection_equals_dense(device):
    cfg = synth.Config("dense", 8, 2, 64, "bf16", 4, 30, (4, 4), 30, 12, 4, n_seq=2)
    inp = synth.generate(cfg, 5)
    sel = np.tile(np.arange(4, dtype=np.int32), (2, 1))
    keep = np.tile(np.arange(1, 31, dtype=np.int32), (8, 1))
    say("K = N, B = C")
    o, lse = _run_gpu(inp, sel, keep, cfg, 3)
    ro, rlse = _oracle(inp, sel, keep, cfg)
    _compare(o, lse, ro, rlse, cfg, "dense")


def test_rerun_is_bitwise_identical(device):
    cfg = synth.config("s8")
    inp = synth.generate(cfg, 2)
    sel, keep = synth.random_page_table(cfg, 2)
    say("s8 rerun determinism")
    a, la = _run_gpu(inp, sel, keep, cfg, 0)
    b, lb = _run_gpu(inp, sel, keep, cfg, 0)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_many_sequences_take_several_launches(device):
    """More sequences than one launch carries (64): the later launches
    address their sequences and split partials by offset.  Mixed K_s,
    including 0 and N, through the planner and a forced split count."""
    ks = tuple((3 * s) % 7 for s in range(70))           # 0 .. 6 chunks of 6
    cfg = synth.Config("seq70", 14, 2, 128, "bf16", 6, 40, ks, 17, 24, 8, n_seq=70)
    inp = synth.generate(cfg, 4)
    sel, keep = synth.random_page_table(cfg, 4)
    ro, rlse = _oracle(inp, sel, keep, cfg)
    for ns in (0, 3):
        say(f"70 sequences, num_splits={ns}")
        o, lse = _run_gpu(inp, sel, keep, cfg, ns)
        _compare(o, lse, ro, rlse, cfg, f"70 sequences splits {ns}")


FORCED = [(d, rows) for d in (64, 128) for rows in (128, 256)]


@pytest.mark.parametrize("d,rows", FORCED, ids=[f"d{d}_rows{r}" for d, r in FORCED])
def test_forced_workgroup_shapes(device, d, rows):
    """Every bf16 kernel instance (4- and 8-wave workgroups, d = 64 and 128)
    on splits of many tiles: one split of 14 tiles and two of 7 refill the
    row table (4 tiles for 4-wave workgroups, 8 for 8-wave), and the last
    chunk is partial, so a split holds absent rows."""
    from diffusion_long_context_amd import _lib as L
    import torch
    cfg = synth.Config("forced", 14, 2, d, "bf16", 8, 100, (8,), 100, 40, 8, last_chunk=60)
    inp = synth.generate(cfg, 6)
    sel, keep = synth.random_page_table(cfg, 6)
    assert (keep == -1).any()
    ro, rlse = _oracle(inp, sel, keep, cfg)
    for ns in (1, 2, 5):
        say(f"d={d} rows={rows} num_splits={ns}")
        call = L.Decode(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(sel), dev(keep),
                        cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale,
                        num_splits=ns, q_rows_per_wg=rows)
        o, lse = call()
        torch.cuda.synchronize()
        _compare(host(o), host(lse), ro, rlse, cfg, f"d={d} rows={rows} splits {ns}")


def test_planner_plan_d64(device):
    """The planner's own plan at d = 64 on a multi-sequence shape (48/8
    heads, L_d = 64, B = 128, K = 32, 4 sequences: 256-row workgroups, 4
    splits of 17 tiles).  Both workgroup shapes at d = 64, forced, run in
    test_forced_workgroup_shapes."""
    from diffusion_long_context_amd import _lib as L
    cfg = synth.Config("d64_auto", 48, 8, 64, "bf16", 32, 128, (32, 32, 32, 32), 128, 64, 8, n_seq=4)
    splits, tps, _, rows = L.decode_plan(cfg.k_per_seq, cfg.b, cfg.l_d, cfg.h_q, cfg.h_kv, cfg.d, 1,
                                         with_rows=True)
    say(f"d64 auto plan: rows {rows}, splits {splits}, tiles per split {tps}")
    inp = synth.generate(cfg, 7)
    sel, keep = synth.random_page_table(cfg, 7)
    heads = [0, 5, 6, 23, 47]
    ro, rlse = _oracle(inp, sel, keep, cfg, heads=heads)
    o, lse = _run_gpu(inp, sel, keep, cfg, 0)
    _compare(o, lse, ro, rlse, cfg, "d64 auto plan", heads=heads)


def test_no_chunk_selected_with_null_tables(device):
    """Every K_s = 0: the decode is attention over the response rows alone,
    and chunk_slot, sel_chunk and keep_rows may be NULL."""
    import ctypes
    import torch
    from diffusion_long_context_amd import _lib as L
    cfg = synth.Config("k0null", 28, 4, 128, "bf16", 3, 64, (0, 0), 8, 70, 8, n_seq=2)
    inp = synth.generate(cfg, 8)
    sel = np.zeros((2, 0), np.int32)
    keep = np.zeros((cfg.n_slots, cfg.b), np.int32)
    ro, rlse = _oracle(inp, sel, keep, cfg)
    pool_k, pool_v = dev(inp.pool_k), dev(inp.pool_v)
    q, kr, vr = dev(inp.q), dev(inp.k_resp), dev(inp.v_resp)
    pool = L.make_pool(pool_k, pool_v)
    ks = (ctypes.c_int32 * 2)(0, 0)
    pt = L.PageTable(None, None, None, ctypes.cast(ks, ctypes.c_void_p), cfg.n_chunks, 0, cfg.b, 0)
    for ns in (0, 1, 2):
        opts = L.DecodeOpts(ns, 0)
        need = L.lib.pdllm_split_attn_decode_ex_workspace(ctypes.byref(pool), ctypes.byref(pt), 2, cfg.l_d,
                                                          cfg.h_q, ctypes.byref(opts))
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((2, cfg.h_q, cfg.l_d), dtype=torch.float32, device=q.device)
        say(f"K=0 with NULL index tables, num_splits={ns}")
        st = L.lib.pdllm_split_attn_decode_ex(ctypes.byref(pool), ctypes.byref(pt), q.data_ptr(), kr.data_ptr(),
                                              vr.data_ptr(), 2, cfg.l_d, cfg.h_q, cfg.scale, ctypes.byref(opts),
                                              o.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(),
                                              torch.cuda.current_stream().cuda_stream)
        assert st == 0, L.lib.pdllm_last_error()
        torch.cuda.synchronize()
        _compare(host(o), host(lse), ro, rlse, cfg, f"K=0 NULL tables splits {ns}")


SMALL_LD = [
    # (name, config, forced split counts): a workgroup of 256 query rows whose
    # last four wavefronts hold none (L_d * G <= 128) splits into computing
    # and loading wavefronts; splits of 17 tiles refill the row table
    ("ld16", synth.Config("ld16", 14, 2, 128, "bf16", 8, 128, (8,), 128, 16, 8), (0, 1, 3)),
    ("ld9_partial", synth.Config("ld9", 14, 2, 128, "bf16", 8, 100, (8,), 100, 9, 8, last_chunk=60), (0, 1, 2)),
    ("ld16_d64_seq70", synth.Config("ld16s", 14, 2, 64, "bf16", 6, 64, tuple(1 + (5 * s) % 6 for s in range(70)),
                                    64, 16, 8, n_seq=70), (0, 2)),
    ("ld40_two_tiles", synth.Config("ld40", 14, 2, 128, "bf16", 6, 64, (6,), 64, 40, 8), (0, 1)),
]


@pytest.mark.parametrize("name,cfg,splits", SMALL_LD, ids=[c[0] for c in SMALL_LD])
def test_small_window_loader_wavefronts(device, name, cfg, splits):
    """Small L_d: the workgroup's wavefronts without query rows load the
    tiles for the others (three staging sets), with absent rows (a partial
    last chunk), d = 64, more sequences than one launch, and a second query
    tile of 24 rows (L_d = 40: the first tile computes on all wavefronts,
    the second splits).  Two calls give identical bits."""
    inp = synth.generate(cfg, 11)
    sel, keep = synth.random_page_table(cfg, 11)
    ro, rlse = _oracle(inp, sel, keep, cfg)
    for ns in splits:
        say(f"{name}: num_splits={ns}")
        o, lse = _run_gpu(inp, sel, keep, cfg, ns)
        _compare(o, lse, ro, rlse, cfg, f"{name} splits {ns}")
        o2, lse2 = _run_gpu(inp, sel, keep, cfg, ns)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "second call differs"
