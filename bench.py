"""Benchmark of the chunk-sparse attention path on one MI355X.

One step is one pass of the whole path over the 32K-prefix workload
(28 query / 4 KV heads, d = 128, bf16; 128 chunks of 256 tokens + BOS in a
randomly permuted pool; K = 16 chunks, B = 256 rows kept, L_d = 256 decode
rows; scoring window = the first 64 decode rows):

  1. chunk-local attention over all 128 chunks with fused per-key scoring
     (pdllm_chunk_prefill_score: prefill kernel + key-score finalize),
  2. top-B rows per chunk (pdllm_select_topB),
  3. top-K chunks over the given chunk scores (pdllm_select_topK),
  4. split-KV decode attention over the selected page table, with the
     log-sum-exp merge (pdllm_split_attn_decode).

Inputs are seeded synthetic data already resident in HBM.  The JSON line
reports algorithmic TFLOP/s of the step (QK^T + PV of the chunk attention,
QK^T of the window scoring, QK^T + PV of the decode), per-stage times from
HIP events on the launch stream, the roofline of the dominant kernel, and
the fp64 oracle timed on the host's cores on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--decode-only", action="store_true",
                   help="time only the decode call (diagnostic; not the headline step)")
    return p.parse_args()


def workload_counts(cfg):
    """Algorithmic FLOPs and HBM bytes of each stage of one step."""
    n, r, hq, hk, d, w = cfg.n_slots, cfg.rows, cfg.h_q, cfg.h_kv, cfg.d, cfg.w
    e = 2  # bf16 bytes
    n_kv = [k * (cfg.b + 1) + cfg.l_d for k in cfg.k_per_seq]
    flops = {
        "prefill": 4.0 * n * r * r * hq * d + 2.0 * n * w * r * hq * d,
        "select_topb": 0.0,
        "select_topk": 0.0,
        "decode": sum(4.0 * cfg.l_d * hq * d * x for x in n_kv),
    }
    bytes_ = {
        # q_chunk + o_chunk + the chunks' pool K/V + query window + key scores
        "prefill": 2.0 * n * r * hq * d * e + 2.0 * n * r * hk * d * e + cfg.n_seq * w * hq * d * e
                   + 4.0 * n * r,
        "select_topb": 4.0 * n * r + 4.0 * n * cfg.b,
        "select_topk": 4.0 * cfg.n_seq * cfg.n_chunks + 4.0 * cfg.n_seq * cfg.k_max,
        # q + kept pool K/V rows (BOS included) + response K/V + o
        "decode": sum(2.0 * cfg.l_d * hq * d * e + 2.0 * x * hk * d * e for x in n_kv),
    }
    return flops, bytes_


def cpu_baseline(cfg, inp, sel, keep):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    the full decode call and 8 of the 128 chunks of the prefill side."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    chunks = list(range(0, cfg.n_slots, cfg.n_slots // 8))[:8]
    t0 = time.perf_counter()
    oracle.chunk_prefill_score(inp.pool_k, inp.pool_v, inp.chunk_slot, inp.q_chunk, inp.q_win,
                               cfg.n_chunks, cfg.scale, chunks=chunks)
    t1 = time.perf_counter()
    oracle.split_attn_decode(inp.pool_k, inp.pool_v, inp.chunk_slot, sel, keep, cfg.k_per_seq, inp.q,
                             inp.k_resp, inp.v_resp, cfg.scale)
    t2 = time.perf_counter()
    flops, _ = workload_counts(cfg)
    f = flops["prefill"] * len(chunks) / cfg.n_slots + flops["decode"]
    return {"value": f / (t2 - t0) / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle: prefill side on {len(chunks)} of {cfg.n_slots} chunks "
                      f"({t1 - t0:.2f} s) + one full decode call ({t2 - t1:.2f} s)",
            "seconds": t2 - t0}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path is measured on a single MI355X "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from diffusion_long_context_amd import _lib as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config("s32")
    inp = synth.generate(cfg, args.seed, with_q_chunk=True)

    def to_dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    pool_k, pool_v = to_dev(inp.pool_k), to_dev(inp.pool_v)
    chunk_slot, chunk_score = to_dev(inp.chunk_slot), to_dev(inp.chunk_score)
    q_chunk, q_win = to_dev(inp.q_chunk), to_dev(inp.q_win)
    q, k_resp, v_resp = to_dev(inp.q), to_dev(inp.k_resp), to_dev(inp.v_resp)
    o_chunk = torch.empty_like(q_chunk)
    key_score = torch.empty((cfg.n_slots, cfg.rows), dtype=torch.float32, device=dev)
    ws_prefill = torch.empty(L.lib.pdllm_prefill_score_workspace(cfg.n_slots, cfg.h_kv, cfg.rows),
                             dtype=torch.uint8, device=dev)
    keep = torch.empty((cfg.n_slots, cfg.b), dtype=torch.int32, device=dev)
    sel = torch.empty((cfg.n_seq, cfg.k_max), dtype=torch.int32, device=dev)
    decode = L.Decode(pool_k, pool_v, chunk_slot, sel, keep, cfg.k_per_seq, q, k_resp, v_resp, cfg.scale)

    def stage_prefill():
        L.chunk_prefill_score(pool_k, pool_v, chunk_slot, q_chunk, q_win, cfg.n_chunks, cfg.scale,
                              o_chunk=o_chunk, key_score=key_score, workspace=ws_prefill)

    stages = [("prefill", stage_prefill),
              ("select_topb", lambda: L.select_topb(key_score, cfg.b, keep_rows=keep)),
              ("select_topk", lambda: L.select_topk(chunk_score, cfg.k_per_seq, cfg.k_max, sel_chunk=sel)),
              ("decode", lambda: decode())]
    if args.decode_only:
        for _, fn in stages[:3]:
            fn()
        stages = stages[3:]

    for _ in range(args.warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        for j, (_, fn) in enumerate(stages):
            fn()
            ev[k][j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    stage_ms = {name: float(np.mean([ev[k][j].elapsed_time(ev[k][j + 1]) for k in range(args.steps)]))
                for j, (name, _) in enumerate(stages)}
    step_ms = float(np.mean([ev[k][0].elapsed_time(ev[k][-1]) for k in range(args.steps)]))

    flops, bytes_ = workload_counts(cfg)
    names = [n for n, _ in stages]
    step_flops = sum(flops[n] for n in names)
    value = step_flops / (step_ms * 1e-3) / 1e12

    def roof(name):
        t = stage_ms[name] * 1e-3
        ai = flops[name] / max(bytes_[name], 1.0)
        hbm_bound = ai < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if hbm_bound:
            ach = bytes_[name] / t / 1e9
            return {"kernel": name, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": bytes_[name],
                    "us": stage_ms[name] * 1e3, "mfma_frac": flops[name] / t / 1e12 / BF16_PEAK_TFLOPS}
        ach = flops[name] / t / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / BF16_PEAK_TFLOPS, "traffic": None, "algorithmic_flops": flops[name],
                "us": stage_ms[name] * 1e3, "hbm_frac": bytes_[name] / t / 1e9 / HBM_PEAK_GBS}

    dominant = max((n for n in names if flops[n] > 0), key=lambda n: stage_ms[n])
    out = {
        "metric": "split-KV chunk attention TFLOP/s + μs/step, 32K prefix; % of bf16 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": step_ms, "us_per_step": step_ms * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, numpy PCG64)",
        "config": {"workload": "32K prefix: 128 chunks x (256+BOS), 28/4 heads, d=128, K=16, B=256, "
                               "L_d=256, window 64; prefill side + top-B + top-K + split decode, 1 layer",
                   "global_batch": cfg.n_seq, "seq_len": cfg.n_chunks * cfg.chunk + cfg.l_d},
        "stage_us": {n: stage_ms[n] * 1e3 for n in names},
        "roofline": roof(dominant),
        "rooflines": {n: roof(n) for n in names if flops[n] > 0},
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        sel_h, keep_h = sel.cpu().numpy(), keep.cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(cfg, inp, sel_h, keep_h)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
