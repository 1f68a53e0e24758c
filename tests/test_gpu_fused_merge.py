"""GPU parity of the decode whose splits are merged inside the decode launch
(pdllm_decode_opts.merge 2 and 3: float32 or bf16 partials exchanged through
one XCD's L2), through the C ABI: against the fp64 oracle and the separate
merge kernel, on the 32K workload, forced workgroup shapes and split counts,
partial chunks (absent rows), and more sequences than one launch carries.
Repeated calls give identical bits, and each call leaves the workspace's
synchronisation words at zero for the next."""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, max_abs, say

pytestmark = pytest.mark.gpu


def _calls(cfg, seed, merge, num_splits=0, rows=0):
    import torch
    from diffusion_long_context_amd import _lib as L
    inp = synth.generate(cfg, seed)
    sel, keep = synth.random_page_table(cfg, seed)
    args = (dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(sel), dev(keep), cfg.k_per_seq,
            dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    call = L.Decode(*args, num_splits=num_splits, q_rows_per_wg=rows, merge=merge)
    # sync words: started, exited, one arrival count per (sequence, kv head,
    # query tile) group of a launch, then the claim counts (checked: the words
    # that are sync words whichever workgroup shape the planner picks)
    groups = min(cfg.n_seq, 64) * cfg.h_kv * -(-cfg.l_d * (cfg.h_q // cfg.h_kv) // 256)
    outs = []
    for _ in range(2):
        o, lse = call()
        torch.cuda.synchronize()
        outs.append((host(o), host(lse)))
        head = call.workspace[:4 * (2 + groups)].view(torch.int32).cpu().numpy()
        assert not head.any(), f"sync words left non-zero: {np.flatnonzero(head)[:8]}"
    sep = L.Decode(*args, num_splits=num_splits, q_rows_per_wg=rows, merge=1)
    o_sep, _ = sep()
    torch.cuda.synchronize()
    return inp, sel, keep, outs, host(o_sep)


CASES = [
    ("s32", synth.config("s32"), 0, 0, [0, 6, 7, 13, 27]),
    ("s32_splits23", synth.config("s32"), 23, 0, [3, 20]),
    ("forced128_partial", synth.Config("p", 14, 2, 128, "bf16", 8, 100, (8,), 100, 40, 8, last_chunk=60), 5, 128,
     None),
    ("d64", synth.Config("d64", 8, 2, 64, "bf16", 6, 64, (5,), 40, 50, 8), 3, 0, None),
    ("seq70", synth.Config("seq70", 14, 2, 128, "bf16", 6, 40, tuple((3 * s) % 7 for s in range(70)), 17, 24, 8,
                           n_seq=70), 3, 0, None),
]


@pytest.mark.parametrize("merge", [2, 3])
@pytest.mark.parametrize("name,cfg,ns,rows,heads", CASES, ids=[c[0] for c in CASES])
def test_in_kernel_merge(device, name, cfg, ns, rows, heads, merge):
    say(f"in-kernel merge {merge}: {name}, num_splits={ns}, rows={rows}")
    inp, sel, keep, outs, o_sep = _calls(cfg, 1, merge, ns, rows)
    (o, lse), (o2, lse2) = outs
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "second call differs"
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq, inp.q,
                                        inp.k_resp, inp.v_resp, cfg.scale, heads=heads)
    if heads is not None:
        o, lse, o_sep = o[:, :, heads], lse[:, heads], o_sep[:, :, heads]
        ro, rlse = ro[:, :, heads], rlse[:, heads]
    r, m = assert_close(o, ro, "bf16", f"{name} merge {merge}")
    ml = max_abs(lse, rlse)
    assert ml <= TOL["bf16"]["lse"], f"lse {ml:.2e}"
    # against the separate merge kernel (bf16 partials): within the bf16 output budget
    r2, m2 = assert_close(o, o_sep, "bf16", f"{name}: merge {merge} against merge 1")
    say(f"  oracle rel-L2 {r:.2e} max-abs {m:.2e} lse {ml:.2e}; vs separate merge rel-L2 {r2:.2e}")


@pytest.mark.parametrize("name,cfg,ns,rows,heads", CASES, ids=[c[0] for c in CASES])
def test_separate_merge_f32_partials(device, name, cfg, ns, rows, heads):
    """merge 4: the separate merge kernel over float32 partials (the output
    rounded once, at the merge) -- against the oracle, and against merge 1's
    bf16 partials; two calls give identical bits."""
    import torch
    from diffusion_long_context_amd import _lib as L
    say(f"separate merge, float32 partials: {name}, num_splits={ns}, rows={rows}")
    inp = synth.generate(cfg, 1)
    sel, keep = synth.random_page_table(cfg, 1)
    args = (dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(sel), dev(keep), cfg.k_per_seq,
            dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    call = L.Decode(*args, num_splits=ns, q_rows_per_wg=rows, merge=4)
    outs = []
    for _ in range(2):
        o, lse = call()
        torch.cuda.synchronize()
        outs.append((host(o), host(lse)))
    (o, lse), (o2, lse2) = outs
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "second call differs"
    o_sep, _ = L.Decode(*args, num_splits=ns, q_rows_per_wg=rows, merge=1)()
    torch.cuda.synchronize()
    o_sep = host(o_sep)
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq, inp.q,
                                        inp.k_resp, inp.v_resp, cfg.scale, heads=heads)
    if heads is not None:
        o, lse, o_sep = o[:, :, heads], lse[:, heads], o_sep[:, :, heads]
        ro, rlse = ro[:, :, heads], rlse[:, heads]
    r, m = assert_close(o, ro, "bf16", f"{name} merge 4")
    ml = max_abs(lse, rlse)
    assert ml <= TOL["bf16"]["lse"], f"lse {ml:.2e}"
    r1, m1 = assert_close(o_sep, ro, "bf16", f"{name} merge 1")
    say(f"  oracle rel-L2: float32 partials {r:.2e} (max-abs {m:.2e}), bf16 partials {r1:.2e} (max-abs {m1:.2e})")
