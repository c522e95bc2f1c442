#!/usr/bin/env python3
"""MSA decode benchmark on one MI355X.

One step = one msa_decode call: one pass of the whole decode hot path over
one batch (index scores + block max-pool, block top-k, sparse attention).  Inputs are resident in HBM before timing starts.  To
keep the 256 MB Infinity Cache from serving the scan, the step rotates over
several copies of the caches at different addresses ("layers"), as a real
model's decode would over its layers.

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded on
the launch stream inside the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA decode queries/s + achieved HBM GB/s (% of peak) at 256K ctx, FP8 KV"
HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, topk_counts):
    """Bytes the method must move per step (decode rows, R = 1)."""
    import numpy as np
    ik_tok = {2: 128, 3: 72, 0: 512}[w.index_k_dtype]
    kv_tok = {2: 256, 3: 144, 0: 1024}[w.kv_dtype]  # K+V per token per head
    lens = w.seq_lens.astype(np.int64)
    nb = (lens + 127) // 128
    rows, G, MB = w.rows, w.num_groups, w.max_blocks
    qb = 2 if w.q_dtype == 1 else 4
    index = (int(lens.sum()) * ik_tok + rows * G * 128 * qb + int(nb.sum()) * 4
             + rows * G * MB * 4)
    topk = rows * G * MB * 4 + rows * G * w.top_k * 4
    attend = (int(topk_counts) * kv_tok + rows * w.num_q_heads * 128 * qb * 2
              + rows * G * w.top_k * (4 + 4))
    return index, topk, attend


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="fp8_long",
                    choices=["fp8_long", "fp8_b32", "nvfp4_512k", "fp8_256k"])
    ap.add_argument("--layers", type=int, default=4, help="cache copies rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py runs on one GPU only: this build has no multi-GPU path "
            "(see DESIGN.md for how it would shard); run with --gpus 1")
        sys.exit(2)

    import numpy as np
    import torch

    import decode_msa_index_amd as msa
    import synth
    from tests import parity

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    msa.lib()
    t0 = time.time()
    if args.workload == "fp8_256k":
        w = synth.make("fp8_256k", seed=0x4D5341 + 5, seq_lens=[262144] * 8,
                       q_dtype=synth.BF16, kv_dtype=synth.FP8, plant_per_seq=8)
        w.recipe = "8 seqs x 262144 tokens, as fp8_long otherwise"
    else:
        w = getattr(synth, args.workload)()
    log(f"[bench] generated {w.name} in {time.time() - t0:.1f}s: {w.recipe}")

    dws = [parity.DeviceWorkload(w)]
    for _ in range(1, args.layers):
        d = parity.DeviceWorkload.__new__(parity.DeviceWorkload)
        d.__dict__.update(dws[0].__dict__)
        d.ik_data = dws[0].ik_data.clone()
        d.kv_data = dws[0].kv_data.clone()
        d.ik_scales = None if dws[0].ik_scales is None else dws[0].ik_scales.clone()
        d.kv_scales = None if dws[0].kv_scales is None else dws[0].kv_scales.clone()
        d.ws_attend = dws[0].ws_attend.clone()
        dws.append(d)
    torch.cuda.synchronize()
    log(f"[bench] {args.layers} cache copies resident; "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    # ---- timed region 1: whole decode steps (msa_decode) ----
    for i in range(args.warmup):
        dws[i % len(dws)].decode(with_scores=False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        dws[i % len(dws)].decode(with_scores=False)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = t_total * 1e3 / args.steps

    # ---- timed region 2: the dominant kernel (index scan) per launch, HIP
    # events on the launch stream ----
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.warmup):
        dws[i % len(dws)].index_scores()
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][0].record()
        dws[i % len(dws)].index_scores()
        evs[i][1].record()
    torch.cuda.synchronize()
    k_idx = np.array([e[0].elapsed_time(e[1]) for e in evs])
    k_topk = np.array([0.0])
    k_att = np.array([0.0])
    dws[0].decode(with_scores=True)
    torch.cuda.synchronize()

    topk = dws[0].topk.cpu().numpy()
    sel_tokens = 0
    for r in range(w.rows):
        L = int(w.seq_lens[r])
        for g in range(w.num_groups):
            for j in topk[r, g]:
                if j >= 0:
                    sel_tokens += min(128, L - 128 * int(j))
    b_idx, b_topk, b_att = algorithmic_bytes(w, sel_tokens)
    b_step = b_idx + b_topk + b_att
    idx_us = float(np.mean(k_idx)) * 1e3
    achieved = b_idx / (idx_us * 1e-6) / 1e9
    tokens = int(w.seq_lens.astype(np.int64).sum())
    dense_bytes = tokens * (256 if w.kv_dtype == 2 else 144) * w.num_groups
    log(f"[bench] ms/step {ms_step:.4f}; index kernel {idx_us:.1f} us/launch "
        f"({achieved:.0f} GB/s)")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        p = parity.oracle_problem(w, threads)
        reps, t_c0 = 0, time.perf_counter()
        while True:
            oracle.decode(p, w.index_q, w.ik_data, w.ik_scales, w.q, w.kv_data, w.kv_scales,
                          w.block_table, w.seq_lens, w.q_pos)
            reps += 1
            if time.perf_counter() - t_c0 >= args.cpu_seconds:
                break
        t_c = time.perf_counter() - t_c0
        cpu = {"value": reps * w.rows / t_c, "unit": "queries/s",
               "cores": oracle.threads_used(), "kind": "oracle",
               "sample": f"{reps} full decode step(s) of the same {w.rows}-query batch "
                         f"({tokens} cached tokens) in {t_c:.1f}s, fp64"}
        log(f"[bench] oracle: {cpu['value']:.3f} queries/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": w.rows / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "recipe": w.recipe, "batch": w.num_seqs,
            "context_tokens": tokens, "kv_dtype": synth.DTYPE_NAMES[w.kv_dtype],
            "index_k_dtype": synth.DTYPE_NAMES[w.index_k_dtype], "q_heads": w.num_q_heads,
            "kv_groups": w.num_groups, "head_dim": w.head_dim, "block": w.block_size,
            "top_k": w.top_k, "cache_copies": args.layers,
        },
        "hbm_gbps_step": b_step / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": b_step / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "tokens_scanned_per_s": tokens / (ms_step * 1e-3),
        "bytes_per_step": b_step,
        "dense_attention_bytes_ratio": dense_bytes / b_step,
        "kernel_us": {"index_scores": idx_us,
                      "select_attend_and_gaps": ms_step * 1e3 - idx_us},
        "roofline": {"bound": "hbm", "kernel": "index_scores", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None, "bytes_per_launch": b_idx},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
