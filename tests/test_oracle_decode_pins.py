"""Pins of the oracle's decode attention and LSE merge against values fixed
by the mathematics, independent of the oracle's own code:

* brute force with explicit Python loops on tiny inputs,
* the library routine ``torch.nn.functional.scaled_dot_product_attention``
  (fp64, CPU) in the special cases where the chunk-sparse decode reduces to
  plain dense attention (K = N with B = C, and K = 0),
* closed forms (identical keys, one attended row),
* invariants (pool permutation, key shift, value affinity, split count).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _tiny_cfg(**kw):
    base = dict(name="pin", h_q=4, h_kv=2, d=8, dtype="f32", n_chunks=5, chunk=6,
                k_per_seq=(3,), b=4, l_d=3, w=3, n_seq=1)
    base.update(kw)
    return synth.Config(**base)


def _brute_decode(inp, sel, keep, cfg):
    """Loop-by-loop evaluation of the decode definition on tiny inputs."""
    pk, pv = oracle.as_f64(inp.pool_k), oracle.as_f64(inp.pool_v)
    q, kr, vr = oracle.as_f64(inp.q), oracle.as_f64(inp.k_resp), oracle.as_f64(inp.v_resp)
    n_seq, l_d, h_q, d = q.shape
    g_size = cfg.h_q // cfg.h_kv
    o = np.zeros((n_seq, l_d, h_q, d))
    lse = np.zeros((n_seq, h_q, l_d))
    for s in range(n_seq):
        keys, vals = [], []
        for k in range(cfg.k_per_seq[s]):
            c = s * cfg.n_chunks + int(sel[s][k])
            slot = int(inp.chunk_slot[c])
            rows = [0] + [int(x) for x in keep[c]]
            for r in rows:
                keys.append(pk[slot, r])
                vals.append(pv[slot, r])
        for j in range(l_d):
            keys.append(kr[s, j])
            vals.append(vr[s, j])
        for i in range(l_d):
            for h in range(h_q):
                g = h // g_size
                z = []
                for a in range(len(keys)):
                    acc = 0.0
                    for e in range(d):
                        acc += q[s, i, h, e] * keys[a][g, e]
                    z.append(cfg.scale * acc)
                zmax = max(z)
                ex = [math.exp(t - zmax) for t in z]
                tot = sum(ex)
                for e in range(d):
                    o[s, i, h, e] = sum(ex[a] * vals[a][g, e] for a in range(len(keys))) / tot
                lse[s, h, i] = zmax + math.log(tot)
    return o, lse


def _run(inp, sel, keep, cfg):
    return oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep,
                                    cfg.k_per_seq, inp.q, inp.k_resp, inp.v_resp, cfg.scale)


@pytest.mark.parametrize("seed,kw", [
    (0, {}),
    (1, dict(n_seq=2, k_per_seq=(2, 5), b=6)),
    (2, dict(h_q=3, h_kv=1, k_per_seq=(0,), l_d=4)),
    (3, dict(h_q=2, h_kv=2, d=4, chunk=1, b=1, n_chunks=3, k_per_seq=(3,), l_d=1)),
    (4, dict(n_seq=3, k_per_seq=(1, 0, 4), b=0, l_d=2)),
    (5, dict(dtype="bf16", h_q=6, h_kv=3, d=16, k_per_seq=(2,))),
])
def test_decode_matches_brute_force(seed, kw):
    cfg = _tiny_cfg(**kw)
    inp = synth.generate(cfg, seed)
    sel, keep = synth.random_page_table(cfg, seed)
    o, lse = _run(inp, sel, keep, cfg)
    bo, blse = _brute_decode(inp, sel, keep, cfg)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def _sdpa(q, k, v, scale):
    """Library attention, fp64 CPU. q [L][h_q][d], k/v [N][h_kv][d]."""
    h_q, h_kv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(h_q // h_kv, dim=0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(h_q // h_kv, dim=0)[None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return out[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("seed", [0, 7])
def test_full_selection_is_dense_attention(seed):
    """K = N and B = C: the attended set is every row of every chunk plus the
    response, so the result is dense bidirectional attention over the
    concatenation, whatever the pool order."""
    cfg = _tiny_cfg(n_seq=2, k_per_seq=(5, 5), b=6)
    inp = synth.generate(cfg, seed)
    sel = np.tile(np.arange(cfg.n_chunks, dtype=np.int32), (cfg.n_seq, 1))
    keep = np.tile(np.arange(1, cfg.chunk + 1, dtype=np.int32), (cfg.n_slots, 1))
    o, _ = _run(inp, sel, keep, cfg)
    pk, pv = oracle.as_f64(inp.pool_k), oracle.as_f64(inp.pool_v)
    for s in range(cfg.n_seq):
        slots = inp.chunk_slot[s * cfg.n_chunks:(s + 1) * cfg.n_chunks]
        kk = np.concatenate([pk[slots].reshape(-1, cfg.h_kv, cfg.d), oracle.as_f64(inp.k_resp[s])])
        vv = np.concatenate([pv[slots].reshape(-1, cfg.h_kv, cfg.d), oracle.as_f64(inp.v_resp[s])])
        ref = _sdpa(oracle.as_f64(inp.q[s]), kk, vv, cfg.scale)
        np.testing.assert_allclose(o[s], ref, rtol=0, atol=1e-12)


def test_no_chunks_is_response_attention():
    cfg = _tiny_cfg(k_per_seq=(0,), l_d=5)
    inp = synth.generate(cfg, 3)
    sel, keep = synth.random_page_table(cfg, 3)
    o, _ = _run(inp, sel, keep, cfg)
    ref = _sdpa(oracle.as_f64(inp.q[0]), oracle.as_f64(inp.k_resp[0]),
                oracle.as_f64(inp.v_resp[0]), cfg.scale)
    np.testing.assert_allclose(o[0], ref, rtol=0, atol=1e-12)


def test_pool_permutation_invariance():
    cfg = _tiny_cfg(n_seq=2, k_per_seq=(3, 2))
    inp = synth.generate(cfg, 11)
    sel, keep = synth.random_page_table(cfg, 11)
    o1, l1 = _run(inp, sel, keep, cfg)
    perm = np.random.default_rng(5).permutation(cfg.n_slots)   # new slot of old slot
    pk2 = np.empty_like(inp.pool_k)
    pv2 = np.empty_like(inp.pool_v)
    pk2[perm] = inp.pool_k
    pv2[perm] = inp.pool_v
    inp.pool_k, inp.pool_v = pk2, pv2
    inp.chunk_slot = perm[inp.chunk_slot].astype(np.int32)
    o2, l2 = _run(inp, sel, keep, cfg)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_identical_keys_give_mean_of_values():
    """All attended keys equal: softmax is uniform, o = mean(v), and
    lse = scale <q, k> + ln N_kv."""
    cfg = _tiny_cfg(n_seq=2, k_per_seq=(2, 4), b=3, l_d=4)
    inp = synth.generate(cfg, 4)
    sel, keep = synth.random_page_table(cfg, 4)
    kvec = np.random.default_rng(9).standard_normal((cfg.h_kv, cfg.d)).astype(np.float32)
    inp.pool_k[:] = kvec
    inp.k_resp[:] = kvec
    o, lse = _run(inp, sel, keep, cfg)
    for s in range(cfg.n_seq):
        _, vv = oracle.attended_kv(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep,
                                   cfg.k_per_seq[s], s, cfg.n_chunks, inp.k_resp, inp.v_resp)
        n_kv = cfg.k_per_seq[s] * (cfg.b + 1) + cfg.l_d
        assert vv.shape[0] == n_kv
        for h in range(cfg.h_q):
            g = h // (cfg.h_q // cfg.h_kv)
            np.testing.assert_allclose(o[s, :, h], np.broadcast_to(vv[:, g].mean(0), o[s, :, h].shape),
                                       rtol=0, atol=1e-12)
            z = cfg.scale * (oracle.as_f64(inp.q[s, :, h]) @ kvec[g].astype(np.float64))
            np.testing.assert_allclose(lse[s, h], z + math.log(n_kv), rtol=0, atol=1e-12)


def test_single_attended_row_returns_its_value():
    cfg = _tiny_cfg(k_per_seq=(0,), l_d=1)
    inp = synth.generate(cfg, 2)
    sel, keep = synth.random_page_table(cfg, 2)
    o, lse = _run(inp, sel, keep, cfg)
    for h in range(cfg.h_q):
        g = h // (cfg.h_q // cfg.h_kv)
        np.testing.assert_array_equal(o[0, 0, h], oracle.as_f64(inp.v_resp[0, 0, g]))
        z = cfg.scale * float(oracle.as_f64(inp.q[0, 0, h]) @ oracle.as_f64(inp.k_resp[0, 0, g]))
        assert abs(lse[0, h, 0] - z) <= 1e-12


def test_key_shift_and_value_affine():
    cfg = _tiny_cfg(n_seq=1, k_per_seq=(3,), l_d=3)
    inp = synth.generate(cfg, 6)
    sel, keep = synth.random_page_table(cfg, 6)
    o, lse = _run(inp, sel, keep, cfg)
    # key shift: adding one vector c to every key adds scale<q,c> to each z
    cvec = np.random.default_rng(1).standard_normal((cfg.h_kv, cfg.d))
    shifted = synth.generate(cfg, 6)
    shifted.pool_k = (oracle.as_f64(inp.pool_k) + cvec)
    shifted.k_resp = (oracle.as_f64(inp.k_resp) + cvec)
    o2, lse2 = _run(shifted, sel, keep, cfg)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-11)
    for h in range(cfg.h_q):
        g = h // (cfg.h_q // cfg.h_kv)
        dz = cfg.scale * (oracle.as_f64(inp.q[0, :, h]) @ cvec[g])
        np.testing.assert_allclose(lse2[0, h], lse[0, h] + dz, rtol=0, atol=1e-11)
    # value affinity: o(a v + b) = a o(v) + b
    a, bvec = 2.5, np.random.default_rng(2).standard_normal(cfg.d)
    aff = synth.generate(cfg, 6)
    aff.pool_v = a * oracle.as_f64(inp.pool_v) + bvec
    aff.v_resp = a * oracle.as_f64(inp.v_resp) + bvec
    o3, lse3 = _run(aff, sel, keep, cfg)
    np.testing.assert_allclose(o3, a * o + bvec, rtol=0, atol=1e-11)
    np.testing.assert_array_equal(lse3, lse)


@pytest.mark.parametrize("seed", range(4))
def test_split_merge_equals_direct(seed):
    """Any partition of the KV rows, merged by log-sum-exp, equals direct
    attention (empty parts included)."""
    rng = np.random.default_rng(seed)
    m, n, d = 5, 37, 8
    q = rng.standard_normal((m, d))
    k = rng.standard_normal((n, d)) * 3
    v = rng.standard_normal((n, d))
    scale = 0.3
    p, mx, l = oracle.softmax_rows(scale * (q @ k.T))
    direct_o, direct_lse = p @ v, mx + np.log(l)
    for n_parts in (1, 2, 3, 7, 37):
        cuts = np.sort(rng.choice(np.arange(1, n), size=n_parts - 1, replace=False)) if n_parts > 1 else []
        parts = np.split(rng.permutation(n), cuts)
        parts.append(np.array([], dtype=np.int64))          # an empty part
        o, lse = oracle.attention_over_parts(q, k, v, scale, parts)
        np.testing.assert_allclose(o, direct_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, direct_lse, rtol=0, atol=1e-12)
    # the direct result is itself plain library attention
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=scale)[0].numpy()
    np.testing.assert_allclose(direct_o, ref, rtol=0, atol=1e-12)


def test_lse_merge_closed_form():
    """Two parts with lse 0 and ln 3 weigh 1:3."""
    o_parts = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    lse_parts = np.array([[0.0], [math.log(3.0)]])
    o, lse = oracle.lse_merge(o_parts, lse_parts)
    np.testing.assert_allclose(o, [[0.25, 0.75]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, [math.log(4.0)], rtol=0, atol=1e-15)


def test_bf16_decoding_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80, 0x0001], dtype=np.uint16)
    vals = oracle.as_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0
    assert vals[2] == 3.140625
    assert vals[3] == 0.0 and math.copysign(1, vals[4]) == -1.0
    assert math.isinf(vals[5])
    assert vals[6] == 2.0 ** -133          # smallest bf16 subnormal
    # round trip of the generator's rounding for representable values
    x = np.array([1.0, -2.5, 3.140625, 65280.0], dtype=np.float32)
    np.testing.assert_array_equal(oracle.as_f64(synth.f32_to_bf16_bits(x)), x.astype(np.float64))
