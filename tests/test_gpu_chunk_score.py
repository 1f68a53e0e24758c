"""GPU parity of pdllm_chunk_score (per-token log-probabilities over the
vocabulary, summed into s_I, s_P and s per chunk) against the fp64 oracle."""
import math

import numpy as np
import pytest

import oracle
import synth
from _parity import dev, host, say

pytestmark = pytest.mark.gpu


def _gpu(logits, target, n_q, n_p, dtype):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(logits).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        t = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    vocab = logits.shape[2]
    return t, torch.from_numpy(target).cuda(), vocab


def _score(logits, target, n_q, n_p, dtype, vocab=None):
    import torch
    from diffusion_long_context_amd import _lib as L
    t, tg, width = _gpu(logits, target, n_q, n_p, dtype)
    v = width if vocab is None else vocab
    out = L.chunk_score(t[..., :v] if v != width else t, tg, n_q, n_p)
    torch.cuda.synchronize()
    return tuple(host(x).astype(np.float64) for x in out)


def _bound(lp_rows):
    """Worst-case float32 error of a chunk's score: per row 4e-5 (the
    vocabulary sum's rounding, taken sequentially over about 600 terms per
    thread, then combined in a tree), plus the rounding of the row sum."""
    return 4e-5 * lp_rows.shape[1] + 1e-6 * np.abs(lp_rows).sum(axis=1)


CASES = [
    ("v1000", 3, 4, 5, 1000, "bf16", 0),
    ("v1000_f32", 3, 4, 5, 1000, "f32", 0),
    ("v4099_ragged", 2, 3, 2, 4099, "bf16", 4104),
    ("v4099_f32_ragged", 2, 3, 2, 4099, "f32", 4100),
    ("v777_padded_rows", 2, 2, 3, 777, "bf16", 832),
    ("v152064_full", 2, 3, 3, 152064, "bf16", 0),
    ("query_only", 3, 5, 0, 2000, "bf16", 0),
    ("pseudo_only", 3, 0, 5, 2000, "bf16", 0),
    ("vocab1", 2, 2, 2, 1, "f32", 4),
]


@pytest.mark.parametrize("name,n_c,n_q,n_p,vocab,dtype,stride", CASES, ids=[c[0] for c in CASES])
def test_chunk_score_matches_oracle(device, name, n_c, n_q, n_p, vocab, dtype, stride):
    logits, target = synth.chunk_logits(n_c, n_q, n_p, vocab, seed=3, dtype=dtype, stride=stride)
    say(f"chunk score {name}")
    s_i, s_p, s = _score(logits, target, n_q, n_p, dtype, vocab=vocab)
    r_i, r_p, r = oracle.chunk_scores(logits[..., :vocab], target, n_q, n_p)
    lp = oracle.token_log_probs(logits[..., :vocab], target).reshape(n_c, n_q + n_p)
    tol_i, tol_p = _bound(lp[:, :n_q]), _bound(lp[:, n_q:])
    assert np.all(np.abs(s_i - r_i) <= tol_i), (s_i - r_i, tol_i)
    assert np.all(np.abs(s_p - r_p) <= tol_p), (s_p - r_p, tol_p)
    assert np.all(np.abs(s - r) <= tol_i + tol_p + 1e-6 * np.abs(r))
    assert np.array_equal(s.astype(np.float32), (s_i.astype(np.float32) + s_p.astype(np.float32)))
    again = _score(logits, target, n_q, n_p, dtype, vocab=vocab)
    assert all(np.array_equal(a, b) for a, b in zip(again, (s_i, s_p, s))), "not reproducible"


def test_uniform_logits_closed_form(device):
    """Equal logits: every log-probability is -ln V exactly up to float32."""
    n_c, n_q, n_p, v = 2, 3, 4, 50000
    logits = np.full((n_c, n_q + n_p, v), 1.5, dtype=np.float32)
    target = np.zeros((n_c, n_q + n_p), dtype=np.int32)
    s_i, s_p, s = _score(logits, target, n_q, n_p, "f32")
    assert np.allclose(s_i, n_q * math.log(v), rtol=2e-6, atol=0)
    assert np.allclose(s_p, -n_p * math.log(v), rtol=2e-6, atol=0)


def test_scores_feed_top_k(device):
    """The GPU's chunk scores select the same chunks on the GPU and in the
    oracle (same float32 array, bit-exact), and the same as the fp64 scores
    wherever the cut is not a near-tie."""
    import torch
    from diffusion_long_context_amd import _lib as L
    n_c, n_q, n_p, v, k = 40, 4, 4, 3000, 7
    logits, target = synth.chunk_logits(n_c, n_q, n_p, v, seed=4)
    s = _score(logits, target, n_q, n_p, "bf16")[2]
    s32 = s.astype(np.float32)[None, :]
    sel = host(L.select_topk(torch.from_numpy(s32).cuda(), [k], k))
    assert np.array_equal(sel, oracle.select_topk(s32, [k], k))
    r = oracle.chunk_scores(logits, target, n_q, n_p)[2]
    srt = np.sort(r)[::-1]
    if srt[k - 1] - srt[k] > 4 * np.abs(s - r).max():
        assert np.array_equal(sel, oracle.select_topk(r[None, :], [k], k))


def test_no_scored_rows_give_zero_scores(device):
    import torch
    from diffusion_long_context_amd import _lib as L
    logits = torch.empty((3, 0, 64), dtype=torch.bfloat16, device="cuda")
    target = torch.empty((3, 0), dtype=torch.int32, device="cuda")
    out = tuple(torch.full((3,), 7.0, device="cuda") for _ in range(3))
    L.chunk_score(logits, target, 0, 0, out=out)
    torch.cuda.synchronize()
    assert all(np.array_equal(host(x), np.zeros(3)) for x in out)
