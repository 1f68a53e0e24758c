"""Write the Tiny workload's oracle results to ``tiny_seed0.json``.

Calls only the seeded generator (``synth``) and the fp64 oracle
(``oracle``).  The stored values are regression pins of the oracle for the
Tiny configuration (1/1 heads, d=64, fp32, 8 chunks of 64 + BOS, K=2, B=16,
32 decode rows that are also the scoring window, seed 0): selected chunks,
kept rows, and summary statistics of the key scores and the decode output.

Usage:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth   # noqa: E402


def tiny_chain(seed=0):
    cfg = synth.config("tiny")
    inp = synth.generate(cfg, seed, with_q_chunk=True)
    o_chunk, key_score = oracle.chunk_prefill_score(
        inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win, cfg.n_chunks, cfg.scale)
    keep = oracle.select_topb(key_score.astype(np.float32), cfg.b)
    sel = oracle.select_topk(inp.chunk_score, cfg.k_per_seq, cfg.k_max)
    o, lse = oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep,
                                      cfg.k_per_seq, inp.q, inp.k_resp, inp.v_resp, cfg.scale)
    return dict(o_chunk=o_chunk, key_score=key_score, keep_rows=keep, sel_chunk=sel, o=o, lse=lse)


def summary(res):
    return {
        "sel_chunk": res["sel_chunk"].tolist(),
        "keep_rows": res["keep_rows"].tolist(),
        "key_score_sum": float(res["key_score"].sum()),
        "key_score_first_chunk": [float(x) for x in res["key_score"][0]],
        "o_chunk_sum": float(res["o_chunk"].sum()),
        "o_chunk_sumsq": float((res["o_chunk"] ** 2).sum()),
        "o_sum": float(res["o"].sum()),
        "o_sumsq": float((res["o"] ** 2).sum()),
        "o_row0": [float(x) for x in res["o"][0, 0, 0]],
        "lse": [float(x) for x in res["lse"][0, 0]],
    }


if __name__ == "__main__":
    out = summary(tiny_chain(0))
    out["_about"] = ("fp64 oracle on the seeded Tiny workload (seed 0); written by "
                     "tests/golden/make_golden.py")
    with open(os.path.join(HERE, "tiny_seed0.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("wrote tiny_seed0.json")
