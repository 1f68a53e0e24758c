"""GPU: the attended pool rows resolved once (pdllm_resolve_rows) give the
same decode, bit for bit, as the index tables, in both decode kernels (split
plans and the decode without splits), with absent kept rows, compacted slots,
sequences with no selected chunk and more sequences than one launch; and the
resolved entries equal the oracle's attended rows."""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, max_abs, say

pytestmark = pytest.mark.gpu

CASES = [
    # (name, config, (num_splits, q_rows_per_wg) pairs)
    ("s8", synth.config("s8"), ((0, 0), (0, 256), (3, 0))),
    ("f32", synth.config("f32"), ((0, 0), (0, 32))),
    ("s32", synth.config("s32"), ((0, 0), (0, 32), (23, 0))),
    ("absent", synth.Config("abs", 14, 2, 128, "bf16", 8, 100, (8,), 100, 40, 8, last_chunk=60),
     ((0, 0), (2, 128), (0, 32))),
    ("d64_seq70", synth.Config("s70", 14, 2, 64, "bf16", 6, 40, tuple((3 * s) % 7 for s in range(70)), 17, 24, 8,
                               n_seq=70), ((0, 0), (3, 0), (0, 32))),
]


@pytest.mark.parametrize("name,cfg,runs", CASES, ids=[c[0] for c in CASES])
def test_resolved_rows_match_index_tables(device, name, cfg, runs):
    import torch
    from diffusion_long_context_amd import _lib as L
    inp = synth.generate(cfg, 3)
    sel, keep = synth.random_page_table(cfg, 3)
    args = [dev(x) for x in (inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep)]
    rest = (cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    ro = rl = None
    for ns, rows in runs:
        say(f"{name}: num_splits={ns} q_rows_per_wg={rows}, tables then resolved rows")
        o_t, l_t = L.Decode(*args, *rest, num_splits=ns, q_rows_per_wg=rows)()
        d = L.Decode(*args, *rest, num_splits=ns, q_rows_per_wg=rows, resolve=True)
        o_r, l_r = d()
        torch.cuda.synchronize()
        assert torch.equal(o_r, o_t) and torch.equal(l_r, l_t), f"{name} {ns} {rows}: resolved rows differ"
        if ro is None and name not in ("s32",):
            ro, rl = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                              inp.q, inp.k_resp, inp.v_resp, cfg.scale)
        if ro is not None:
            assert_close(host(o_r), ro, cfg.dtype, f"{name} resolved")
            assert max_abs(host(l_r), rl) <= TOL[cfg.dtype]["lse"]
    # the resolved entries against the oracle's attended rows (slot, row)
    rows_h = d.rows.cpu().numpy().astype(np.int64).reshape(cfg.n_seq, cfg.k_max, cfg.b + 1) \
        if cfg.k_max else None
    if rows_h is not None:
        pk = inp.pool_k
        ps_slot, ps_row = pk.shape[1] * pk.shape[2] * pk.shape[3], pk.shape[2] * pk.shape[3]
        for s in range(min(cfg.n_seq, 5)):
            for k in range(cfg.k_per_seq[s]):
                c = int(sel[s, k])
                slot = int(inp.chunk_slot[s * cfg.n_chunks + c])
                for r in range(cfg.b + 1):
                    e = int(rows_h[s, k, r])
                    kr = -2 if r == 0 else int(keep[s * cfg.n_chunks + c, r - 1])
                    absent = r > 0 and kr < 0
                    want = (slot * ps_slot + (0 if r == 0 or absent else kr) * ps_row) // 8
                    assert (e & 0x7fffffff) == want and (e < 0) == absent, (s, k, r)


def test_resolved_rows_compacted_slots(device):
    """Compacted slots (kept row i at slot row 1 + i; keep_rows marks the
    absent rows): resolved rows give the gathering decode's bits."""
    import torch
    from diffusion_long_context_amd import _lib as L
    cfg = synth.Config("cmp", 14, 2, 128, "bf16", 8, 100, (5,), 64, 20, 8, last_chunk=40)
    inp = synth.generate(cfg, 9)
    sel, keep = synth.random_page_table(cfg, 9)
    ck, cv = L.compact_kept_rows(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(keep))
    rest = (cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    for rows in (0, 32):
        o_t, l_t = L.Decode(ck, cv, dev(inp.chunk_slot), dev(sel), dev(keep), *rest, compacted=True,
                            q_rows_per_wg=rows)()
        o_r, l_r = L.Decode(ck, cv, dev(inp.chunk_slot), dev(sel), dev(keep), *rest, compacted=True,
                            q_rows_per_wg=rows, resolve=True)()
        torch.cuda.synchronize()
        assert torch.equal(o_r, o_t) and torch.equal(l_r, l_t), f"compacted rows={rows}: resolved rows differ"
