"""GPU parity of the decode without kv splits (pdllm_decode_opts.q_rows_per_wg
= 32: one workgroup per 32 query rows over every kv row, no partials) against
the fp64 oracle, through the C ABI: the 8K / 32K full-step layer / 32K
workloads whole, the 128K batch on sampled heads, and small shapes with
d = 64, mixed K_s (0 included), b = 0, absent kept rows, compacted slots, a
query block that ends inside a tile, fewer kv tiles than wavefronts, a pool
table at the row cap, and more sequences than one launch carries."""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, max_abs, say

pytestmark = pytest.mark.gpu

WS = 32


def _run(inp, sel, keep, cfg, compacted=False, pool=None):
    import torch
    from diffusion_long_context_amd import _lib as L
    pk, pv = pool if pool is not None else (inp.pool_k, inp.pool_v)
    call = L.Decode(dev(pk), dev(pv), dev(inp.chunk_slot), dev(sel), dev(keep), cfg.k_per_seq, dev(inp.q),
                    dev(inp.k_resp), dev(inp.v_resp), cfg.scale, q_rows_per_wg=WS, compacted=compacted)
    o, lse = call()
    torch.cuda.synchronize()
    return host(o), host(lse)


def _check(o, lse, ro, rlse, cfg, what, heads=None):
    if heads is not None:
        o, ro, lse, rlse = o[:, :, heads], ro[:, :, heads], lse[:, heads], rlse[:, heads]
    r, m = assert_close(o, ro, cfg.dtype, what)
    ml = max_abs(lse, rlse)
    assert ml <= TOL[cfg.dtype]["lse"], f"{what}: lse max-abs {ml:.3e}"
    say(f"  {what}: rel-L2 {r:.2e} max-abs {m:.2e} lse {ml:.2e}")


@pytest.mark.parametrize("name", ["s8", "f32", "s32"])
def test_full_size(device, name):
    cfg = synth.config(name)
    inp = synth.generate(cfg, 2)
    sel, keep = synth.random_page_table(cfg, 2)
    say(f"{name}: oracle")
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                        inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    say(f"{name}: gpu, 32-row decode")
    o, lse = _run(inp, sel, keep, cfg)
    _check(o, lse, ro, rlse, cfg, f"{name} 32-row")
    o2, lse2 = _run(inp, sel, keep, cfg)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "second call differs"


def test_s128_sampled_heads(device):
    cfg = synth.config("s128")
    say("s128: generating inputs")
    inp = synth.generate(cfg, 0)
    sel, keep = synth.random_page_table(cfg, 0)
    heads = [0, 6, 13, 21, 27]
    say("s128: oracle on sampled heads")
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                        inp.q, inp.k_resp, inp.v_resp, cfg.scale, heads=heads)
    say("s128: gpu, 32-row decode")
    o, lse = _run(inp, sel, keep, cfg)
    _check(o, lse, ro, rlse, cfg, "s128 32-row", heads=heads)


SHAPES = [
    # (name, config): ragged query blocks (L_d * G not a multiple of 32),
    # boundary tiles that hold pool and response rows, partial last tiles
    ("g7_d128", synth.Config("g7", 7, 1, 128, "bf16", 6, 40, (3,), 17, 33, 4)),
    ("d64_multi_k0", synth.Config("d64m", 4, 2, 64, "bf16", 4, 31, (4, 0, 1), 9, 70, 4, n_seq=3)),
    ("b0", synth.Config("b0", 3, 3, 64, "bf16", 7, 16, (5,), 0, 5, 4)),
    ("one_row", synth.Config("one", 8, 2, 128, "bf16", 3, 8, (0,), 2, 1, 4)),
    ("absent_rows", synth.Config("abs", 14, 2, 128, "bf16", 8, 100, (8,), 100, 40, 8, last_chunk=60)),
    ("absent_d64", synth.Config("abs64", 14, 2, 64, "bf16", 8, 100, (8,), 100, 9, 8, last_chunk=60)),
    ("pool_rows_at_cap", synth.Config("cap", 8, 1, 128, "bf16", 40, 160, (32,), 151, 24, 8)),
    ("seq70", synth.Config("seq70", 14, 2, 128, "bf16", 6, 40, tuple((3 * s) % 7 for s in range(70)), 17, 24, 8,
                           n_seq=70)),
]


@pytest.mark.parametrize("name,cfg", SHAPES, ids=[s[0] for s in SHAPES])
def test_shapes(device, name, cfg):
    inp = synth.generate(cfg, 5)
    sel, keep = synth.random_page_table(cfg, 5)
    if name == "pool_rows_at_cap":
        assert cfg.k_per_seq[0] * (cfg.b + 1) == 4864
    if name.startswith("absent"):
        assert (keep == -1).any()
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                        inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    say(f"{name}: 32-row decode")
    o, lse = _run(inp, sel, keep, cfg)
    _check(o, lse, ro, rlse, cfg, f"{name} 32-row")


def test_compacted_slots(device):
    """Kept rows compacted to rows 1..b of each slot (keep_rows only marks
    absent rows): the same attended rows as the gathering decode."""
    cfg = synth.Config("cmp", 14, 2, 128, "bf16", 8, 100, (5,), 64, 20, 8, last_chunk=40)
    inp = synth.generate(cfg, 9)
    sel, keep = synth.random_page_table(cfg, 9)
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                        inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    ck, cv, _ = oracle.compact_kept_rows(inp.pool_k, inp.pool_v, inp.chunk_slot, keep, cfg.n_slots)
    say("compacted slots: 32-row decode")
    o, lse = _run(inp, sel, keep, cfg, compacted=True, pool=(ck, cv))
    _check(o, lse, ro, rlse, cfg, "compacted 32-row")
