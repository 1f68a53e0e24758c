"""The comparators that put the chunk-sparse decode in context, on the same
GPU and through the same C ABI: (i) dense bidirectional attention over every
token of a 32K-prefix step (L_p + L_d = 33,024 rows), the decode with no
selected chunk and all tokens as query/response rows; (ii) gather-to-
contiguous then attention: pdllm_gather_kept_kv copies each sequence's
attended pool rows into one run, and a decode over that run (one compacted
chunk per sequence) attends them.  The gather is bit-exact against the
oracle's attended rows, attention over the gathered run equals the in-place
decode bit for bit and the oracle within tolerance, and the dense path
matches the oracle on sampled rows at full size."""
import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, max_abs, say

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


GATHER = [("small", synth.Config("g", 14, 2, 128, "bf16", 7, 40, (3, 5), 17, 20, 8, n_seq=2)),
          ("d64", synth.Config("g", 8, 4, 64, "bf16", 5, 33, (5,), 32, 9, 8)),
          ("f32", synth.config("f32"))]


@pytest.mark.parametrize("name,cfg", GATHER, ids=[g[0] for g in GATHER])
def test_gather_then_attention(device, name, cfg):
    import torch
    from diffusion_long_context_amd import _lib as L
    inp = synth.generate(cfg, 2)
    sel, keep = synth.random_page_table(cfg, 2)
    pk, pv, slot = dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot)
    say(f"gather {name}")
    gk, gv = L.gather_kept_kv(pk, pv, slot, dev(sel), dev(keep), cfg.k_per_seq)
    torch.cuda.synchronize()
    gk_h, gv_h = _bits(gk), _bits(gv)
    per = cfg.b + 1
    for s, ks in enumerate(cfg.k_per_seq):
        slots, rows = oracle.attended_pool_rows(inp.chunk_slot, sel, keep, ks, s, cfg.n_chunks)
        got_k = gk_h[s * cfg.k_max: s * cfg.k_max + ks].reshape(ks * per, cfg.h_kv, cfg.d)
        got_v = gv_h[s * cfg.k_max: s * cfg.k_max + ks].reshape(ks * per, cfg.h_kv, cfg.d)
        assert np.array_equal(got_k, inp.pool_k[slots, rows]), f"{name}: gathered K of sequence {s}"
        assert np.array_equal(got_v, inp.pool_v[slots, rows]), f"{name}: gathered V of sequence {s}"
    # attention over each sequence's gathered run, as one compacted chunk of
    # K_s (b + 1) rows, equals the in-place decode (uniform K_s only)
    if len(set(cfg.k_per_seq)) != 1:
        return
    ks = cfg.k_per_seq[0]
    run_k = gk.view(cfg.n_seq, cfg.k_max * per, cfg.h_kv, cfg.d)
    run_v = gv.view(cfg.n_seq, cfg.k_max * per, cfg.h_kv, cfg.d)
    one = torch.zeros((cfg.n_seq, 1), dtype=torch.int32, device=pk.device)
    seq_slot = torch.arange(cfg.n_seq, dtype=torch.int32, device=pk.device)
    rest = (dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    contiguous = L.Decode(run_k, run_v, seq_slot, one, None, [1] * cfg.n_seq, *rest, b=ks * per - 1)
    in_place = L.Decode(pk, pv, slot, dev(sel), dev(keep), cfg.k_per_seq, *rest)
    o_c, l_c = contiguous()
    o_p, l_p = in_place()
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p), f"{name}: contiguous attention differs from in place"
    heads = [0, 5, cfg.h_q - 1]
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq, inp.q,
                                        inp.k_resp, inp.v_resp, cfg.scale, heads=heads)
    r, m = assert_close(host(o_c)[:, :, heads], ro[:, :, heads], "bf16", f"{name} contiguous vs oracle")
    say(f"  {name}: gathered rows exact; contiguous == in place; oracle rel-L2 {r:.2e} max-abs {m:.2e}")


def test_dense_attention_32k_step(device):
    """(i) at full size: 33,024 query rows (28 heads) attend all 33,024 rows
    (4 KV heads, d = 128), bf16; sampled rows against the oracle."""
    import torch
    from diffusion_long_context_amd import _lib as L
    n = 32768 + 256
    cfg = synth.Config("dense32k", 28, 4, 128, "bf16", 1, 1, (0,), 0, n, 1)
    say("dense 32K step: generating")
    inp = synth.generate(cfg, 0)
    sel = np.zeros((1, 0), np.int32)
    keep = np.zeros((1, 0), np.int32)
    say("dense 32K step: gpu")
    call = L.Decode(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(sel), dev(keep), [0], dev(inp.q),
                    dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    o, lse = call()
    torch.cuda.synchronize()
    o_h, lse_h = host(o), host(lse)
    assert np.isfinite(o_h).all()
    k = oracle.as_f64(inp.k_resp[0])
    v = oracle.as_f64(inp.v_resp[0])
    everything = [np.arange(n)]
    errs = []
    for i in (0, 1, 4095, 16511, n - 1):
        for h in (0, 6, 7, 27):
            g = h // (cfg.h_q // cfg.h_kv)
            ro, rl = oracle.attention_over_parts(oracle.as_f64(inp.q[0, i, h])[None], k[:, g], v[:, g], cfg.scale,
                                                 everything)
            errs.append(max_abs(o_h[0, i, h], ro[0]))
            assert max_abs(o_h[0, i, h], ro[0]) <= TOL["bf16"]["max_abs"], f"row {i} head {h}"
            assert abs(lse_h[0, h, i] - rl[0]) <= TOL["bf16"]["lse"], f"lse row {i} head {h}"
    say(f"  dense 32K step: 20 sampled rows, max-abs {max(errs):.2e}")
