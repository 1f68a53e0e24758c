"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch each of them.  This shows the pins are sensitive to a wrong
head map, a wrong softmax axis, a dropped BOS row, a dropped scale, a wrong
merge weight and a wrong tie rule -- not only to gross breakage."""
import numpy as np
import pytest

import oracle
import oracle.reference as ref
import test_oracle_decode_pins as dp
import test_oracle_prefill_select_pins as sp


def _fails(fn, *args):
    """The pin must reject the planted mistake (a failed comparison, or a
    shape error where the mistake changes an output's shape)."""
    with pytest.raises((AssertionError, ValueError)):
        fn(*args)


def test_wrong_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(ref, "kv_head_of", lambda h, group: h % group)
    _fails(dp.test_full_selection_is_dense_attention, 0)
    _fails(sp.test_prefill_output_is_per_chunk_sdpa, 0, {})
    _fails(sp.test_head_mapping_probe)


def test_wrong_softmax_axis_is_caught(monkeypatch):
    def bad(z):
        m = np.max(z, axis=0, keepdims=True)
        e = np.exp(z - m)
        l = np.sum(e, axis=0, keepdims=True)
        return e / l, m[0], l[0]
    monkeypatch.setattr(ref, "softmax_rows", bad)
    _fails(dp.test_decode_matches_brute_force, 0, {})
    _fails(sp.test_scores_sum_to_window_rows_times_heads)


def test_dropped_bos_is_caught(monkeypatch):
    orig = ref.attended_pool_rows

    def no_bos(*a, **k):
        slots, rows = orig(*a, **k)
        keep = rows != 0
        return slots[keep], rows[keep]
    monkeypatch.setattr(ref, "attended_pool_rows", no_bos)
    _fails(dp.test_full_selection_is_dense_attention, 0)
    _fails(dp.test_decode_matches_brute_force, 0, {})


def test_dropped_scale_is_caught(monkeypatch):
    orig = ref.split_attn_decode
    monkeypatch.setattr(oracle, "split_attn_decode",
                        lambda *a, **k: orig(*a[:-1], 1.0, **k))
    _fails(dp.test_decode_matches_brute_force, 0, {})


def test_wrong_merge_weight_is_caught(monkeypatch):
    def bad(o_parts, lse_parts):
        m = np.max(lse_parts, axis=0)
        w = np.exp(lse_parts - m[None])
        total = np.sum(w, axis=0)
        o = np.sum(o_parts, axis=0) / o_parts.shape[0]     # plain mean of parts
        return o, m + np.log(total)
    monkeypatch.setattr(ref, "lse_merge", bad)
    monkeypatch.setattr(oracle, "lse_merge", bad)
    _fails(dp.test_split_merge_equals_direct, 0)
    _fails(dp.test_lse_merge_closed_form)


def test_wrong_tie_rule_is_caught(monkeypatch):
    def bad(value, index):
        return (0, -value, -index) if value == value else (1, 0.0, -index)
    monkeypatch.setattr(ref, "_rank_key", bad)
    _fails(sp.test_topb_special_values)
    _fails(sp.test_topb_matches_lexsort, 0)


import test_oracle_chunk_score_pins as cp


def test_wrong_log_softmax_axis_is_caught(monkeypatch):
    def bad(logits, target):
        z = oracle.as_f64(logits).reshape(-1, logits.shape[-1])
        t = np.asarray(target).reshape(-1)
        m = z.max(axis=0)                              # over rows, not the vocabulary
        lse = m + np.log(np.exp(z - m[None, :]).sum(axis=0))
        return z[np.arange(z.shape[0]), t] - lse[t]
    monkeypatch.setattr(ref, "token_log_probs", bad)
    _fails(cp.test_chunk_score_is_sum_of_row_log_probs, 3, 6)


def test_target_off_by_one_is_caught(monkeypatch):
    orig = ref.token_log_probs
    monkeypatch.setattr(ref, "token_log_probs",
                        lambda z, t: orig(z, np.minimum(np.asarray(t) + 1, z.shape[-1] - 1)))
    monkeypatch.setattr(oracle, "token_log_probs", ref.token_log_probs)
    _fails(cp.test_two_token_closed_form)
    _fails(cp.test_chunk_score_signs_and_rows)


def test_flipped_or_swapped_score_parts_are_caught(monkeypatch):
    orig = ref.chunk_scores
    monkeypatch.setattr(ref, "chunk_scores", lambda *a: (lambda r: (-r[0], r[1], r[1] - r[0]))(orig(*a)))
    monkeypatch.setattr(oracle, "chunk_scores", ref.chunk_scores)
    _fails(cp.test_chunk_score_signs_and_rows)
    monkeypatch.setattr(ref, "chunk_scores",
                        lambda z, t, nq, npp: orig(z[:, ::-1], t[:, ::-1], nq, npp))
    monkeypatch.setattr(oracle, "chunk_scores", ref.chunk_scores)
    _fails(cp.test_chunk_score_signs_and_rows)
