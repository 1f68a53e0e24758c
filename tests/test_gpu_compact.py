"""GPU parity of the compacted kept-row layout through the C ABI:
pdllm_compact_kept_rows against the oracle's compaction (bit-exact: it is a
copy), and pdllm_split_attn_decode over compacted slots (rows_compacted = 1)
against the same call over the whole-chunk pool with keep_rows (bit-identical:
the attended rows and their order are the same) and against the fp64 oracle
(the bf16 / f32 tolerances).  Covers f32 and bf16, d = 64 and 128, padded
destination strides, b = 0, b = C, ragged tails, several sequences, and the
32K workload with B = 128."""
import numpy as np
import pytest

import oracle
import synth
from _parity import assert_close, dev, host, max_abs, say, TOL

pytestmark = pytest.mark.gpu


def _bits(t):
    """Raw bits of a device tensor as a numpy array (uint16 for bf16)."""
    import torch
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _compact_gpu(inp, keep, n_chunks, pad_rows=0, pad_row=0):
    """Compaction into a destination with pad_rows extra rows per slot and
    pad_row extra elements per row (strides padded), filled with a marker."""
    import torch
    from diffusion_long_context_amd import _lib as L
    pk, pv = dev(inp.pool_k), dev(inp.pool_v)
    n_slots, _, h_kv, d = pk.shape
    b = keep.shape[1]
    big = torch.full((n_slots, b + 1 + pad_rows, h_kv * d + pad_row), -7.0, dtype=pk.dtype, device=pk.device)
    big_v = torch.full_like(big, -9.0)
    dk = big[:, :, :h_kv * d].unflatten(2, (h_kv, d))
    dv = big_v[:, :, :h_kv * d].unflatten(2, (h_kv, d))
    L.compact_kept_rows(pk, pv, dev(inp.chunk_slot), dev(keep), dk, dv)
    torch.cuda.synchronize()
    return dk, dv, big, big_v


CASES = [
    # (name, config): b = the config's kept-row count
    ("tiny_f32", synth.config("tiny")),
    ("f32_d32_b0", synth.Config("c", 6, 2, 32, "f32", 5, 20, (3,), 0, 9, 4)),
    ("bf16_d64_ragged", synth.Config("c", 4, 2, 64, "bf16", 7, 37, (4, 2), 13, 11, 4, n_seq=2)),
    ("bf16_d128_all_rows", synth.Config("c", 28, 4, 128, "bf16", 4, 64, (3,), 64, 20, 4)),
    ("bf16_d128_s8", synth.config("s8")),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_compaction_is_bit_exact(device, name, cfg):
    inp = synth.generate(cfg, 0)
    _, keep = synth.random_page_table(cfg, 0)
    b = cfg.b
    n_chunks = cfg.n_slots
    ref_k, ref_v, written = oracle.compact_kept_rows(inp.pool_k, inp.pool_v, inp.chunk_slot, keep, n_chunks)
    for pad_rows, pad_row in ((0, 0), (2, 8)):
        say(f"compact {name} b={b} pad=({pad_rows},{pad_row})")
        dk, dv, big, big_v = _compact_gpu(inp, keep, n_chunks, pad_rows, pad_row)
        k, v = _bits(dk[:, :b + 1]), _bits(dv[:, :b + 1])
        assert np.array_equal(k[written], ref_k[written]), f"{name}: K differs"
        assert np.array_equal(v[written], ref_v[written]), f"{name}: V differs"
        # nothing outside rows 0..b of the listed slots was written
        h_kv, d = cfg.h_kv, cfg.d
        if pad_rows:
            assert (host(big[:, b + 1:]) == -7.0).all() and (host(big_v[:, b + 1:]) == -9.0).all()
        if pad_row:
            assert (host(big[:, :, h_kv * d:]) == -7.0).all() and (host(big_v[:, :, h_kv * d:]) == -9.0).all()


def test_compaction_of_part_of_the_chunks(device):
    """Only the listed chunks' slots are written."""
    cfg = synth.Config("c", 8, 2, 128, "bf16", 9, 30, (3,), 7, 5, 4)
    inp = synth.generate(cfg, 4)
    _, keep = synth.random_page_table(cfg, 4)
    n_chunks = 5
    import torch
    from diffusion_long_context_amd import _lib as L
    pk, pv = dev(inp.pool_k), dev(inp.pool_v)
    dk = torch.full((cfg.n_slots, cfg.b + 1, cfg.h_kv, cfg.d), 3.0, dtype=pk.dtype, device=pk.device)
    dv = torch.full_like(dk, 3.0)
    say("compact 5 of 9 chunks")
    L.compact_kept_rows(pk, pv, dev(inp.chunk_slot), dev(keep[:n_chunks]), dk, dv)
    torch.cuda.synchronize()
    ref_k, ref_v, written = oracle.compact_kept_rows(inp.pool_k, inp.pool_v, inp.chunk_slot, keep, n_chunks)
    k, v = _bits(dk), _bits(dv)
    assert np.array_equal(k[written], ref_k[written]) and np.array_equal(v[written], ref_v[written])
    assert (host(dk[torch.from_numpy(~written.any(axis=1)).to(dk.device)]) == 3.0).all()


def _decodes(cfg, seed, num_splits_list, heads=None):
    """Decode over the whole pool with keep_rows, then over the compacted
    slots; both through the C ABI.  Returns the oracle result too."""
    import torch
    from diffusion_long_context_amd import _lib as L
    inp = synth.generate(cfg, seed)
    sel, keep = synth.random_page_table(cfg, seed)
    pk, pv = dev(inp.pool_k), dev(inp.pool_v)
    slot = dev(inp.chunk_slot)
    ck, cv = L.compact_kept_rows(pk, pv, slot, dev(keep))
    args = (slot, dev(sel))
    rest = (cfg.k_per_seq, dev(inp.q), dev(inp.k_resp), dev(inp.v_resp), cfg.scale)
    ro, rlse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq,
                                        inp.q, inp.k_resp, inp.v_resp, cfg.scale, heads=heads)
    out = []
    for ns in num_splits_list:
        say(f"{cfg.name} seed={seed} splits={ns}: gather, then compacted")
        o_g, l_g = L.Decode(pk, pv, *args, dev(keep), *rest, num_splits=ns)()
        o_c, l_c = L.Decode(ck, cv, *args, None, *rest, num_splits=ns, b=cfg.b)()
        torch.cuda.synchronize()
        out.append((ns, host(o_g), host(l_g), host(o_c), host(l_c)))
    return out, ro, rlse


SMALL = [
    ("f32_d64", synth.Config("f32_d64", 2, 1, 64, "f32", 8, 64, (2,), 16, 32, 4)),
    ("bf16_d64_multi", synth.Config("bf16_d64_multi", 4, 2, 64, "bf16", 4, 31, (4, 0, 1), 9, 70, 4, n_seq=3)),
    ("bf16_d128_b0", synth.Config("bf16_d128_b0", 14, 2, 128, "bf16", 7, 16, (5,), 0, 33, 4)),
    ("bf16_d128", synth.Config("bf16_d128", 28, 4, 128, "bf16", 6, 40, (3,), 17, 45, 4)),
]


@pytest.mark.parametrize("name,cfg", SMALL, ids=[c[0] for c in SMALL])
def test_decode_over_compacted_slots(device, name, cfg):
    for seed in (0, 1):
        runs, ro, rlse = _decodes(cfg, seed, (0, 1, 3))
        for ns, o_g, l_g, o_c, l_c in runs:
            assert np.array_equal(o_c, o_g) and np.array_equal(l_c, l_g), f"{name} splits {ns}: not identical"
            r, m = assert_close(o_c, ro, cfg.dtype, f"{name} seed {seed} splits {ns}")
            assert max_abs(l_c, rlse) <= TOL[cfg.dtype]["lse"]


def test_decode_over_compacted_slots_32k(device):
    """The 32K workload with B = 128: compacted and gathered decodes are
    bit-identical; sampled heads match the oracle."""
    cfg = synth.config("f32")
    heads = [0, 6, 13, 20, 27]
    runs, ro, rlse = _decodes(cfg, 0, (0,), heads=heads)
    for ns, o_g, l_g, o_c, l_c in runs:
        assert np.array_equal(o_c, o_g) and np.array_equal(l_c, l_g)
        assert_close(o_c[:, :, heads], ro[:, :, heads], "bf16", "32K compacted")
        assert max_abs(l_c[:, heads], rlse[:, heads]) <= TOL["bf16"]["lse"]
