"""GPU top-B / top-K selection against the oracle's selection on the same
float32 arrays: bit-exact, including ties, signed zeros, infinities, NaN,
B = 0, B = C, K = 0, K = N and more sequences than one launch carries."""
import numpy as np
import pytest

import oracle
from _parity import dev, say

pytestmark = pytest.mark.gpu


def _topb(ks, b):
    from diffusion_long_context_amd import _lib as L
    import torch
    out = L.select_topb(dev(ks.astype(np.float32)), b)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _topk(cs, kps, k_max):
    from diffusion_long_context_amd import _lib as L
    import torch
    out = L.select_topk(dev(cs.astype(np.float32)), kps, k_max)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("rows,seed", [(257, 0), (257, 1), (65, 2), (33, 3), (4097, 4), (2, 5)])
def test_topb_bit_exact(device, rows, seed):
    rng = np.random.default_rng(seed)
    n_chunks = 37
    ks = rng.integers(0, 9, size=(n_chunks, rows)).astype(np.float32)     # heavy ties
    ks[::3] += rng.standard_normal(ks[::3].shape).astype(np.float32)
    ks[5, 1::7] = -0.0
    ks[6, 2::5] = np.nan
    ks[7, 3::9] = np.inf
    ks[8, 1::4] = -np.inf
    for b in sorted({0, 1, (rows - 1) // 2, rows - 1, min(128, rows - 1)}):
        say(f"top-B rows={rows} b={b}")
        got = _topb(ks, b)
        want = oracle.select_topb(ks, b)
        assert got.shape == want.shape
        assert np.array_equal(got, want), f"rows {rows} b {b}"


def test_topb_engineered_order(device):
    ks = np.array([[9.0, 0.0, -0.0, np.nan, np.inf, -np.inf, 1.0, 0.0, np.nan]], dtype=np.float32)
    for b in range(9):
        assert np.array_equal(_topb(ks, b), oracle.select_topb(ks, b))


@pytest.mark.parametrize("n_seq,n,seed", [(1, 128, 0), (4, 512, 1), (70, 40, 2), (3, 8192, 3), (2, 1, 4)])
def test_topk_bit_exact(device, n_seq, n, seed):
    rng = np.random.default_rng(100 + seed)
    cs = rng.random((n_seq, n), dtype=np.float32)
    cs[:, ::4] = np.round(cs[:, ::4] * 4) / 4               # ties
    if n > 10:
        cs[0, 3] = np.nan
        cs[0, 4] = -0.0
        cs[0, 5] = 0.0
    kps = [int(x) for x in rng.integers(0, n + 1, size=n_seq)]
    kps[0] = n
    if n_seq > 1:
        kps[1] = 0
    k_max = max(kps)
    say(f"top-K n_seq={n_seq} n={n}")
    got = _topk(cs, kps, k_max)
    want = oracle.select_topk(cs, kps, k_max)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n,seed", [(1025, 0), (6000, 1), (8192, 2)])
def test_topk_radix_select_ties(device, n, seed):
    """Above 1024 candidates the selection runs a radix select over the score
    keys: heavy ties (a few distinct scores, so the threshold falls inside a
    tie group, which the lower indices win), NaN, +-0 and +-inf, at K from 1
    to n - 1 -- bit-exact against the oracle."""
    rng = np.random.default_rng(300 + seed)
    cs = rng.integers(0, 6, size=(3, n)).astype(np.float32)
    cs[0, 7::11] = np.nan
    cs[1, 5::13] = -0.0
    cs[1, 6::13] = 0.0
    cs[2, 9::17] = np.inf
    cs[2, 10::19] = -np.inf
    for k in (1, 17, n // 3, n // 2, n - 2, n - 1):
        kps = [k, max(k - 5, 0), min(k + 5, n)]
        say(f"radix top-K n={n} k={kps}")
        got = _topk(cs, kps, max(kps))
        want = oracle.select_topk(cs, kps, max(kps))
        assert np.array_equal(got, want), f"n {n} k {kps}"
