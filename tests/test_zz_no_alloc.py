"""The decode entry point that allocates nothing
(pdllm_split_attn_decode_noalloc), through the C ABI on the GPU: two calls
in a row -- the 8K-prefix workload, then a smaller one, both with split
partials, then the 8K workload's own plan without splits -- each give the same
output and lse as pdllm_split_attn_decode with a caller workspace (bit for
bit: the same kernels and plan) and agree with the fp64 oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from _parity import TOL, assert_close, dev, host, max_abs, say

pytestmark = pytest.mark.gpu


def _noalloc(inp, sel, keep, cfg, num_splits=0):
    import torch
    from diffusion_long_context_amd import _lib as L
    ref = L.Decode(dev(inp.pool_k), dev(inp.pool_v), dev(inp.chunk_slot), dev(sel), dev(keep), cfg.k_per_seq,
                   dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale, num_splits=num_splits)
    o_ref, lse_ref = ref()
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    st = L.lib.pdllm_split_attn_decode_noalloc(
        ctypes.byref(ref.pool), ctypes.byref(ref.pt), ref._keep[3].data_ptr(), ref._keep[4].data_ptr(),
        ref._keep[5].data_ptr(), ref.n_seq, ref.l_d, ref.h_q, ref.scale, num_splits, o.data_ptr(), lse.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.lib.pdllm_last_error()
    torch.cuda.synchronize()
    return o, lse, o_ref, lse_ref, ref.workspace.numel()


def test_noalloc_two_calls_match_workspace_call(device):
    import torch
    # split partials in the scratch array (the 8K workload, 9 forced splits,
    # then a smaller case), then the planner's plan for the 8K workload, the
    # decode without splits, which uses no scratch
    cases = [(synth.config("s8"), 1, 9, True),
             (synth.Config("small", 14, 2, 128, "bf16", 6, 40, (4,), 17, 33, 8), 2, 3, True),
             (synth.config("s8"), 1, 0, False)]
    for cfg, seed, ns, partials in cases:
        inp = synth.generate(cfg, seed)
        sel, keep = synth.random_page_table(cfg, seed)
        say(f"no-allocation decode: {cfg.name}, num_splits={ns}")
        o, lse, o_ref, lse_ref, ws_bytes = _noalloc(inp, sel, keep, cfg, ns)
        assert (ws_bytes > 256) == partials, "the case must (not) use split partials"
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"{cfg.name}: differs from the workspace call"
        ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                            inp.q, inp.k_resp, inp.v_resp, cfg.scale)
        r, m = assert_close(host(o), ro, "bf16", f"{cfg.name} no-allocation decode")
        ml = max_abs(host(lse), rlse)
        assert ml <= TOL["bf16"]["lse"]
        say(f"  {cfg.name}: identical to the workspace call; oracle rel-L2 {r:.2e} max-abs {m:.2e} lse {ml:.2e}")
