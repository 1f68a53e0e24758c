"""Plant plausible mistakes in the oracle (on the CPU) and check that the
pins catch each of them.  This shows the pins are sensitive to a wrong
head map, a wrong softmax axis, a dropped BOS row, a dropped scale, a wrong
merge weight, a wrong tie rule, wrong log-softmax terms and a misplaced BOS
row or slot in the kept-row compaction -- not only to gross breakage."""
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


def test_compaction_without_bos_is_caught(monkeypatch):
    import test_oracle_compact_pins as cp

    def no_bos(pool_k, pool_v, chunk_slot, keep_rows, n_chunks):
        n_slots, _, h_kv, d = pool_k.shape
        b = keep_rows.shape[1]
        k = np.zeros((n_slots, b + 1, h_kv, d), dtype=pool_k.dtype)
        v = np.zeros_like(k)
        written = np.zeros((n_slots, b + 1), dtype=bool)
        for c in range(n_chunks):
            slot = int(chunk_slot[c])
            rows = [int(x) for x in keep_rows[c]] + [0]    # BOS moved behind the kept rows
            k[slot], v[slot] = pool_k[slot, rows], pool_v[slot, rows]
            written[slot] = True
        return k, v, written
    monkeypatch.setattr(oracle, "compact_kept_rows", no_bos)
    _fails(cp.test_compacted_rows_carry_their_source_coordinates, 5)


def test_compaction_into_chunk_index_is_caught(monkeypatch):
    import test_oracle_compact_pins as cp
    orig = ref.compact_kept_rows

    def by_chunk(pool_k, pool_v, chunk_slot, keep_rows, n_chunks):
        # chunk c lands in slot c instead of slot chunk_slot[c]
        k, v, written = orig(pool_k, pool_v, chunk_slot, keep_rows, n_chunks)
        perm = np.asarray(chunk_slot[:n_chunks])
        k2, v2 = np.zeros_like(k), np.zeros_like(v)
        k2[:n_chunks], v2[:n_chunks] = k[perm], v[perm]
        return k2, v2, written
    monkeypatch.setattr(oracle, "compact_kept_rows", by_chunk)
    _fails(cp.test_compacted_rows_carry_their_source_coordinates, 5)


def test_partial_chunk_read_as_whole_is_caught(monkeypatch):
    import test_oracle_partial_pins as pp
    orig = ref.chunk_prefill_score
    monkeypatch.setattr(oracle, "chunk_prefill_score",
                        lambda *a, chunk_rows=None, **k: orig(*a, **k))
    _fails(pp.test_partial_chunk_prefill_is_sdpa_over_its_rows, 0, {})
    orig_b = ref.select_topb
    monkeypatch.setattr(oracle, "select_topb", lambda s, b, chunk_rows=None: orig_b(s, b))
    _fails(pp.test_topb_of_a_partial_chunk, 3)


def test_absent_row_read_as_a_row_is_caught(monkeypatch):
    import test_oracle_partial_pins as pp

    def with_absent(chunk_slot, sel_chunk, keep_rows, k_s, seq, n_chunks_per_seq):
        slots, rows = [], []
        for k in range(k_s):
            c = seq * n_chunks_per_seq + int(sel_chunk[seq][k])
            for r in [0] + [int(x) for x in keep_rows[c]]:       # -1 indexes the slot's last row
                slots.append(int(chunk_slot[c]))
                rows.append(r)
        return np.asarray(slots, dtype=np.int64), np.asarray(rows, dtype=np.int64)
    monkeypatch.setattr(ref, "attended_pool_rows", with_absent)
    _fails(pp.test_decode_skips_absent_rows, 0)
