#!/usr/bin/env python3
"""MSA decode benchmark on one MI355X.

One step = one msa_decode call: one pass of the whole decode hot path over
one batch (index scores + block max-pool, block top-k, sparse attention).
Inputs are resident in HBM before timing starts.  To keep the 256 MB
Infinity Cache from serving the scan, the step rotates over several copies of
the caches at different addresses ("layers"), as a real model's decode would
over its layers.

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded on
the launch stream inside the timed region.  The HBM traffic of the index scan
comes from committed rocprofv3 counter runs (profiles/index_scan_traffic.json)
and is reported only while the scan's sources are unchanged since then.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA decode queries/s + achieved HBM GB/s (% of peak) at 256K ctx, FP8 KV"
HBM_PEAK_GBPS = 8000.0
# sources that determine the index scan kernel's memory traffic
SCAN_SOURCES = ["decode_msa_index_amd/csrc/index_block.hpp",
                "decode_msa_index_amd/csrc/index_scores.hip",
                "decode_msa_index_amd/csrc/device.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def scan_fingerprint() -> str:
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per index-scan launch from the committed counter runs, or
    None when they were taken on another workload or older scan sources."""
    path = os.path.join(ROOT, "profiles", "index_scan_traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("scan_sources_sha256") != scan_fingerprint():
        return None
    return t.get("traffic_bytes_per_launch")


def algorithmic_bytes(w, topk_counts):
    """Bytes the method must move per step: the index keys once per sequence
    (the rows of a sequence share one scan), per-row queries, scores and
    selections, and the selected tokens' K/V per (row, group)."""
    import numpy as np
    ik_tok = {2: 128, 3: 72, 0: 512}[w.index_k_dtype]
    kv_tok = {2: 256, 3: 144, 0: 1024}[w.kv_dtype]  # K+V per token per head
    lens = w.seq_lens.astype(np.int64)
    nb = (lens + 127) // 128
    rows, G, MB = w.rows, w.num_groups, w.max_blocks
    qb = 2 if w.q_dtype == 1 else 4
    # index keys: each physical block once, for the most tokens any sequence
    # sees in it (sequences sharing a prefix share its blocks)
    phys, toks = [], []
    for b in range(w.num_seqs):
        j = np.arange(int(nb[b]))
        phys.append(w.block_table[b, : nb[b]].astype(np.int64))
        toks.append(np.minimum(128, lens[b] - 128 * j))
    seen = np.zeros(w.num_phys_blocks, np.int64)
    if phys:
        np.maximum.at(seen, np.concatenate(phys), np.concatenate(toks))
    index = (int(seen.sum()) * ik_tok + rows * G * 128 * qb + int(nb.sum()) * 4
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
    ap.add_argument("--workload", default="fp8_256k",
                    choices=["fp8_256k", "fp8_long", "fp8_b32", "nvfp4_512k", "spec4_256k",
                             "fp8_share64", "nvfp4_share64", "fp8_dcp45_shard", "prefill_64k",
                             "prefill_16k", "prefill_64k_nvfp4"])
    ap.add_argument("--layers", type=int, default=4, help="cache copies rotated per step")
    ap.add_argument("--share-corr", type=float, default=0.0,
                    help="fp8_share64 / nvfp4_share64 only: correlation of the requests' queries with their "
                         "group's common draw (requests continuing one prompt)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--chain", action="store_true",
                    help="also time the steps as the three-call chain (index scores, block "
                         "top-k, sparse attend)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device-to-device (counter calibration) and exit")
    ap.add_argument("--calibrate-read", action="store_true",
                    help="only time the read probes (the scan's index-key blocks and the "
                         "attention's selected K/V, each with its kernel's access pattern "
                         "and no arithmetic) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py runs on one GPU only: the library has no multi-GPU path; "
            "run with --gpus 1")
        sys.exit(2)
    if args.share_corr and args.workload not in ("fp8_share64", "nvfp4_share64"):
        log("--share-corr applies to the fp8_share64 and nvfp4_share64 workloads only")
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        # a plain copy of known size: it reads and writes 2^30 bytes once, so
        # the HBM counters of this dispatch calibrate FETCH_SIZE / WRITE_SIZE
        a = torch.empty(2**30, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copied 1073741824 bytes")
        return

    import decode_msa_index_amd as msa
    import synth
    from decode_msa_index_amd import harness

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    msa.lib()
    t0 = time.time()
    if args.share_corr:
        w = getattr(synth, args.workload)(share_corr=args.share_corr)
        w.recipe += f"; queries {args.share_corr} x the group's common draw"
    else:
        w = getattr(synth, args.workload)()
    log(f"[bench] generated {w.name} in {time.time() - t0:.1f}s: {w.recipe}")
    if args.calibrate_read:
        return calibrate_read(args, w)
    if w.rows_per_seq >= 16:  # a prefill chunk: its own line (rows/s, MFMA roofline)
        return run_prefill(args, w)

    dws = [harness.DeviceWorkload(w)]
    for _ in range(1, args.layers):
        dws.append(dws[0].copy_with_new_caches())
    torch.cuda.synchronize()
    log(f"[bench] {args.layers} cache copies resident; "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    # ---- timed region 1: whole decode steps (msa_decode), eager ----
    for i in range(args.warmup):
        dws[i % len(dws)].decode(with_scores=False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        dws[i % len(dws)].decode(with_scores=False)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = t_total * 1e3 / args.steps

    # per-step distribution (events around each step; a separate pass)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        dws[i % len(dws)].decode(with_scores=False)
        ev[i][1].record()
    torch.cuda.synchronize()
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])

    # ---- timed region 2: the same steps replayed from a HIP graph ----
    graph_ms = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for d in dws:  # warm the capture stream
                d.decode(with_scores=False)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for d in dws:
                d.decode(with_scores=False)
        reps = max(1, args.steps // len(dws))
        g.replay()
        torch.cuda.synchronize()
        t_g = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t_g) * 1e3 / (reps * len(dws))

    # ---- optional: the same steps as the three-call chain (msa_index_scores,
    # msa_block_topk, msa_sparse_attend), eager ----
    chain_ms = None
    if args.chain:
        for i in range(args.warmup):
            dws[i % len(dws)].chain()
        torch.cuda.synchronize()
        t_c = time.perf_counter()
        for i in range(args.steps):
            dws[i % len(dws)].chain()
        torch.cuda.synchronize()
        chain_ms = (time.perf_counter() - t_c) * 1e3 / args.steps
        log(f"[bench] three-call chain: {chain_ms:.4f} ms per step")

    # ---- timed region 3: the dominant kernel (index scan), launched back to
    # back between two HIP events on the launch stream (the average launch
    # duration, as a kernel trace reports it) ----
    for i in range(args.warmup):
        dws[i % len(dws)].index_scores()
    torch.cuda.synchronize()
    e_idx = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e_idx[0].record()
    for i in range(args.steps):
        dws[i % len(dws)].index_scores()
    e_idx[1].record()
    torch.cuda.synchronize()
    idx_us = e_idx[0].elapsed_time(e_idx[1]) * 1e3 / args.steps
    unshared_us = None
    if w.share_seqs > 1:  # the same scan without the share-group hint
        plain = []
        for d in dws:
            c = harness.DeviceWorkload.__new__(harness.DeviceWorkload)
            c.__dict__.update(d.__dict__)
            c.p = dataclasses.replace(d.p, share_seqs=0)
            plain.append(c)
        for i in range(args.warmup):
            plain[i % len(plain)].index_scores()
        e_idx[0].record()
        for i in range(args.steps):
            plain[i % len(plain)].index_scores()
        e_idx[1].record()
        torch.cuda.synchronize()
        unshared_us = e_idx[0].elapsed_time(e_idx[1]) * 1e3 / args.steps
        log(f"[bench] index scan without the share hint: {unshared_us:.1f} us/launch")
    dws[0].decode(with_scores=True)
    torch.cuda.synchronize()

    topk = dws[0].topk.cpu().numpy()
    sel_tokens = 0
    for r in range(w.rows):
        L = int(w.seq_lens[r // w.rows_per_seq])  # visible keys of row r: t < L, t <= pos
        if w.q_pos is not None:
            L = min(L, int(w.q_pos[r]) + 1)
        for gi in range(w.num_groups):
            for j in topk[r, gi]:
                if j >= 0:
                    sel_tokens += min(128, L - 128 * int(j))
    b_idx, b_topk, b_att = algorithmic_bytes(w, sel_tokens)
    b_step = b_idx + b_topk + b_att
    share_sel = None
    if w.share_seqs > 1:  # selected K/V blocks: requested vs distinct per group
        kv_blk = 2 * 128 * 128 * (1 if w.kv_dtype == 2 else 0.5625)
        req, distinct = 0, set()
        for r in range(w.rows):
            b = r // w.rows_per_seq
            for gi in range(w.num_groups):
                for j in topk[r, gi]:
                    if 0 <= j < w.max_blocks:
                        req += 1
                        distinct.add((gi, int(w.block_table[b, j])))
        share_sel = {"blocks_requested": req, "blocks_distinct": len(distinct),
                     "kv_bytes_requested": req * kv_blk, "kv_bytes_distinct": len(distinct) * kv_blk}
        log(f"[bench] selected K/V blocks: {req} requested, {len(distinct)} distinct "
            f"({req * kv_blk / 1e6:.1f} MB vs {len(distinct) * kv_blk / 1e6:.1f} MB)")
    achieved = b_idx / (idx_us * 1e-6) / 1e9
    tokens = int(w.seq_lens.astype(np.int64).sum())
    dense_bytes = tokens * (256 if w.kv_dtype == 2 else 144) * w.num_groups
    log(f"[bench] ms/step {ms_step:.4f} (p10/p50/p90 {np.percentile(step_ms, 10):.4f}/"
        f"{np.percentile(step_ms, 50):.4f}/{np.percentile(step_ms, 90):.4f}; graph "
        f"{graph_ms if graph_ms is None else round(graph_ms, 4)}); index kernel "
        f"{idx_us:.1f} us/launch ({achieved:.0f} GB/s)")

    # the insert half of the step: each sequence's newest token rewritten
    cw = time_cache_write(w, dws[0], np.arange(w.num_seqs),
                          np.maximum(w.seq_lens.astype(np.int64) - 1, 0))
    log(f"[bench] cache write of {cw['tokens']} tokens: {cw['us_per_launch']:.1f} us")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))

        def time_oracle(nthreads, seconds):
            p = oracle.Problem(**w.problem_fields(), num_threads=nthreads)
            reps, t_c0 = 0, time.perf_counter()
            while True:
                oracle.decode(p, w.index_q, w.ik_data, w.ik_scales, w.q, w.kv_data,
                              w.kv_scales, w.block_table, w.seq_lens, w.q_pos)
                reps += 1
                if time.perf_counter() - t_c0 >= seconds:
                    break
            return reps, time.perf_counter() - t_c0, oracle.threads_used()

        reps, t_c, used = time_oracle(threads, args.cpu_seconds)
        reps1, t_c1, _ = time_oracle(1, max(1.0, args.cpu_seconds / 4))
        cpu = {"value": reps * w.rows / t_c, "unit": "queries/s", "cores": used,
               "kind": "oracle",
               "sample": f"{reps} full decode step(s) of the same {w.rows}-query batch "
                         f"({tokens} cached tokens) in {t_c:.1f}s, fp64, {used} threads",
               "value_1_thread": reps1 * w.rows / t_c1}
        log(f"[bench] oracle: {cpu['value']:.3f} queries/s on {used} threads, "
            f"{cpu['value_1_thread']:.3f} on 1")

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
        "ms_per_step_p10_p50_p90": [float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
        "ms_per_step_graph": graph_ms,
        "ms_per_step_chain": chain_ms,
        "hbm_gbps_step": b_step / (ms_step * 1e-3) / 1e9,
        "hbm_frac_step": b_step / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "tokens_scanned_per_s": tokens / (ms_step * 1e-3),
        "bytes_per_step": b_step,
        "dense_attention_bytes_ratio": dense_bytes / b_step,
        "kernel_us": {"index_scores": idx_us,
                      "select_attend_and_gaps": ms_step * 1e3 - idx_us},
        "roofline": {"bound": "hbm",
                     "kernel": "index_shared_kernel" if w.share_seqs > 1 else "index_mfma_kernel",
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name), "bytes_per_launch": b_idx},
        "cache_write": cw,
        "cpu_baseline": cpu,
    }
    if unshared_us is not None:
        out["kernel_us"]["index_scores_without_share_hint"] = unshared_us
        out["config"]["share_seqs"] = w.share_seqs
    if share_sel is not None:
        out["share_selection"] = share_sel
    print(json.dumps(out), flush=True)


def _time_launches(launch, steps, warmup):
    """Mean time (us) of `steps` launches after `warmup`, from HIP events on
    the current stream."""
    import torch
    for i in range(warmup):
        launch(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def calibrate_read(args, w):
    """Read ceilings of the two memory-bound kernels' access patterns, timed
    with the read probes (libmsa_probe.so), which do no arithmetic:

    * the scan: exactly the index-key blocks the scan reads, in the scan's
      order, one wave per 16 KB block with every load 1 KB of consecutive
      bytes; also over the same blocks in physical order, and with 2 and 4
      blocks in flight per wave (decode workloads, FP8 index keys);
    * NVFP4 index keys: the scan's blocks as the cache stores them (8 KB of
      E2M1 data and 1 KB of scales in two arrays), the data alone, and the
      same bytes as one 9 KB record per block;
    * the attention: the K and V planes of every selected block, one wave per
      (row, group) in selection order, as the one-wave attention launch (512
      or more units) reads them; the attention kernel itself (given the same
      selection) is timed beside it (FP8 caches).

    Decode workloads rotate over --layers cache copies like the decode steps;
    prefill chunks use one copy, like their benchmark line."""
    import ctypes

    import numpy as np
    import torch

    from decode_msa_index_amd import harness
    from decode_msa_index_amd.build import PROBE_LIB

    L = ctypes.CDLL(PROBE_LIB)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    L.msa_probe_read_blocks.restype = ci
    L.msa_probe_read_blocks.argtypes = [vp, vp, ci, ci, vp, vp]
    L.msa_probe_read_kv.restype = ci
    L.msa_probe_read_kv.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, vp, vp]
    L.msa_probe_read_records.restype = ci
    L.msa_probe_read_records.argtypes = [vp, vp, vp, ci, ci, ci, vp, vp]
    stream = torch.cuda.current_stream().cuda_stream
    prefill = w.rows_per_seq >= 16
    layers = 1 if prefill else args.layers
    out = {"calibrate_read": w.name, "cache_copies": layers, "steps": args.steps}

    if w.index_k_dtype == 2 and not prefill:
        nb = (w.seq_lens.astype(np.int64) + 127) // 128
        order = np.concatenate([w.block_table[b, : nb[b]] for b in range(w.num_seqs)]).astype(np.int32)
        n = len(order)
        copies = [harness.dev(w.ik_data)]
        for _ in range(1, layers):
            copies.append(copies[0].clone())
        orders = {"scan order": harness.dev(order), "physical order": harness.dev(np.sort(order))}
        sink = torch.zeros(n, dtype=torch.int32, device="cuda")
        results = []
        for name, o in orders.items():
            for bpw in (1, 2, 4):
                def launch(i):
                    rc = L.msa_probe_read_blocks(copies[i % len(copies)].data_ptr(), o.data_ptr(),
                                                 n, bpw, sink.data_ptr(), stream)
                    assert rc == 0, rc
                us = _time_launches(launch, args.steps, args.warmup)
                gbps = n * 16384 / (us * 1e-6) / 1e9
                log(f"[bench] read probe, {name}, {bpw} block(s) per wave: {us:.2f} us per "
                    f"launch, {gbps:.0f} GB/s ({gbps / HBM_PEAK_GBPS:.3f} of 8 TB/s)")
                results.append({"order": name, "blocks_per_wave": bpw, "us_per_launch": us,
                                "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS})
        out["scan"] = {"bytes_per_launch": n * 16384, "results": results}
        del copies

    if w.index_k_dtype == 3 and not prefill:  # NVFP4 index keys: record layouts
        nb = (w.seq_lens.astype(np.int64) + 127) // 128
        order = np.concatenate([w.block_table[b, : nb[b]] for b in range(w.num_seqs)]).astype(np.int32)
        assert order.min() >= 0 and order.max() < w.num_phys_blocks
        n = len(order)
        P = w.num_phys_blocks
        data = harness.dev(np.ascontiguousarray(w.ik_data.reshape(P, 8192)))
        scl = harness.dev(np.ascontiguousarray(w.ik_scales.reshape(P, 1024)))
        rec9 = torch.cat([data, scl], dim=1).contiguous()  # one 9 KB record per block
        layouts = {"8 KB data + 1 KB scales (the cache's layout)": ([data], [scl], 8, 1),
                   "8 KB data only": ([data], [None], 8, 0),
                   "one 9 KB record per block": ([rec9], [None], 9, 0)}
        for name in layouts:  # rotate over copies like the decode steps
            bases, sides, rk, sk = layouts[name]
            for _ in range(1, layers):
                bases.append(bases[0].clone())
                sides.append(None if sides[0] is None else sides[0].clone())
        o = harness.dev(order)
        sink = torch.zeros(n, dtype=torch.int32, device="cuda")
        results = []
        for name, (bases, sides, rk, sk) in layouts.items():
            def launch(i):
                sd = sides[i % len(sides)]
                rc = L.msa_probe_read_records(bases[i % len(bases)].data_ptr(),
                                              None if sd is None else sd.data_ptr(), o.data_ptr(),
                                              n, rk, sk, sink.data_ptr(), stream)
                assert rc == 0, rc
            us = _time_launches(launch, args.steps, args.warmup)
            nbytes = n * (rk + sk) * 1024
            gbps = nbytes / (us * 1e-6) / 1e9
            log(f"[bench] record probe, {name}: {us:.2f} us per launch, {nbytes / 1e6:.1f} MB, "
                f"{gbps:.0f} GB/s ({gbps / HBM_PEAK_GBPS:.3f} of 8 TB/s)")
            results.append({"layout": name, "us_per_launch": us, "bytes_per_launch": nbytes,
                            "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS})
        out["nvfp4_records"] = {"blocks": n, "results": results}
        del layouts

    if w.kv_dtype == 2 and w.rows * w.num_groups >= 512:  # the one-wave attention launch
        base = harness.DeviceWorkload(w)
        base.index_scores()
        base.block_topk()
        torch.cuda.synchronize()
        dws = [base] + [base.copy_with_new_caches() for _ in range(1, layers)]
        units = w.rows * w.num_groups
        topk = base.topk.cpu().numpy()
        bt = w.block_table
        sel = 0
        for u in range(units):  # blocks the probe reads (valid entries only)
            b = (u // w.num_groups) // w.rows_per_seq
            js = topk.reshape(units, w.top_k)[u]
            js = js[(js >= 0) & (js < w.max_blocks)]
            sel += int(np.count_nonzero((bt[b, js] >= 0) & (bt[b, js] < w.num_phys_blocks)))
        sink = torch.zeros(units, dtype=torch.int32, device="cuda")

        def probe(i):
            d = dws[i % len(dws)]
            rc = L.msa_probe_read_kv(d.kv_data.data_ptr(), base.topk.data_ptr(),
                                     base.block_table.data_ptr(), units, w.top_k, w.num_groups,
                                     w.rows_per_seq, w.max_blocks, w.num_phys_blocks,
                                     sink.data_ptr(), stream)
            assert rc == 0, rc

        def attend(i):
            dws[i % len(dws)].sparse_attend(topk=base.topk)

        us_probe = _time_launches(probe, args.steps, args.warmup)
        us_attend = _time_launches(attend, args.steps, args.warmup)
        nbytes = sel * 2 * 16384
        log(f"[bench] K/V read probe: {sel} selected blocks, {nbytes / 1e6:.1f} MB, "
            f"{us_probe:.1f} us per launch ({nbytes / (us_probe * 1e-6) / 1e9:.0f} GB/s); "
            f"the attention on the same selection: {us_attend:.1f} us")
        out["kv"] = {"selected_blocks": sel, "bytes_per_launch": nbytes,
                     "probe_us_per_launch": us_probe, "attend_us_per_launch": us_attend,
                     "probe_gbps": nbytes / (us_probe * 1e-6) / 1e9}
    print(json.dumps(out), flush=True)


def row_last_key(w, r: int) -> int:
    """The last key query row r sees (negative: none): its position, the
    sequence's end and the block table's reach, whichever comes first."""
    b = r // w.rows_per_seq
    last = min(int(w.seq_lens[b]), w.max_blocks * w.block_size) - 1
    return min(int(w.q_pos[r]), last) if w.q_pos is not None else last


def time_cache_write(w, dw, seqs, positions, reps=20):
    """msa_cache_write of len(positions) new tokens into dw's caches (it
    overwrites those slots; run it after the other timings): the average
    launch of a HIP graph of `reps` launches, and the algorithmic bytes per
    launch -- the new tokens' bf16 (or fp32) K, V and index key read, their
    quantised codes and scales written, positions and table entries read."""
    import numpy as np
    import torch

    import decode_msa_index_amd as msa
    import synth
    from decode_msa_index_amd import harness

    n, G, D, Di = len(positions), w.num_groups, w.head_dim, w.index_dim
    gen = torch.Generator(device="cuda").manual_seed(0x4357)
    tdt = torch.float32 if w.q_dtype == synth.F32 else torch.bfloat16
    idt = torch.float32 if w.index_q_dtype == synth.F32 else torch.bfloat16
    k_new = torch.randn(n, G, D, device="cuda", generator=gen).to(tdt)
    v_new = torch.randn(n, G, D, device="cuda", generator=gen).to(tdt)
    ik_new = torch.randn(n, Di, device="cuda", generator=gen).to(idt)
    seq_t = harness.dev(np.asarray(seqs, np.int32))
    pos_t = harness.dev(np.asarray(positions, np.int32))
    call = lambda: msa.cache_write(dw.p, seq_t, pos_t, k_new, v_new, ik_new, dw.block_table,
                                   dw.kv_data, dw.kv_scales, dw.ik_data, dw.ik_scales)
    # a tiny launch issued from Python would time the host call, not the
    # kernel: `reps` launches are captured in one HIP graph and replayed
    # between two events
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            call()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps

    def coded(elems, dtype):  # bytes of `elems` cached values in `dtype`
        return {0: 4 * elems, 2: elems, 3: elems // 2 + elems // 16}[dtype]

    per_token = (2 * G * D * k_new.element_size() + Di * ik_new.element_size() + 8 + 4
                 + coded(2 * G * D, w.kv_dtype) + coded(Di, w.index_k_dtype))
    kernel = "cache_write_token_kernel" if n < 512 else "cache_write_kernel"  # the library's choice
    return {"kernel": kernel, "tokens": n, "us_per_launch": us,
            "bytes_per_launch": n * per_token,
            "gbps": n * per_token / (us * 1e-6) / 1e9}


def run_prefill(args, w):
    """Chunked prefill (many query rows per sequence): one step = one
    msa_decode call over all rows; the dominant kernel is the MFMA index
    contraction (bf16 MFMA for FP8 index keys, f16 for NVFP4), reported
    against the 2.5 PFLOP/s dense peak both share."""
    import numpy as np
    import torch

    from decode_msa_index_amd import harness

    PEAK_BF16_TFLOPS = 2500.0
    dw = harness.DeviceWorkload(w)
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup)):
        dw.decode(with_scores=False)
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    t_start = time.perf_counter()
    for _ in range(steps):
        dw.decode(with_scores=False)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        dw.index_scores()
        evs[i][1].record()
    torch.cuda.synchronize()
    idx_us = float(np.median([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    # algorithmic flops of the index contraction: every row against its
    # visible keys, G groups x 128 dims, multiply + add
    seen = np.array([row_last_key(w, r) + 1 for r in range(w.rows)], np.int64).clip(0)
    flops = 2.0 * 128 * w.num_groups * float(seen.sum())
    achieved = flops / (idx_us * 1e-6) / 1e12
    log(f"[bench] prefill ms/step {ms_step:.4f}; index contraction {idx_us:.1f} us "
        f"({achieved:.0f} TFLOP/s)")
    # the attention alone on the step's selection (msa_sparse_attend: for
    # chunks of 384+ rows the key-block lists, attention and merge)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        dw.sparse_attend()
        evs[i][1].record()
    torch.cuda.synchronize()
    att_us = float(np.median([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    log(f"[bench] sparse attention on the step's selection: {att_us:.1f} us")
    # the insert half: the chunk's own tokens written into the caches
    cw = time_cache_write(w, dw, np.arange(w.rows) // w.rows_per_seq, w.q_pos)
    log(f"[bench] cache write of {cw['tokens']} tokens: {cw['us_per_launch']:.1f} us "
        f"({cw['gbps']:.0f} GB/s)")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        sample = np.asarray(list(range(0, w.rows, max(1, w.rows // 64)))[:64], np.int64)
        ws = dataclasses.replace(  # the same caches, the sampled query rows
            w, rows_per_seq=len(sample), index_q=np.ascontiguousarray(w.index_q[sample]),
            q=np.ascontiguousarray(w.q[sample]), q_pos=np.ascontiguousarray(w.q_pos[sample]))
        p = oracle.Problem(**ws.problem_fields(), num_threads=threads)
        reps, t_c0 = 0, time.perf_counter()
        while True:
            oracle.decode(p, ws.index_q, ws.ik_data, ws.ik_scales, ws.q, ws.kv_data,
                          ws.kv_scales, ws.block_table, ws.seq_lens, ws.q_pos)
            reps += 1
            if time.perf_counter() - t_c0 >= args.cpu_seconds:
                break
        t_c = time.perf_counter() - t_c0
        cpu = {"value": reps * len(sample) / t_c, "unit": "rows/s",
               "cores": oracle.threads_used(), "kind": "oracle",
               "sample": f"{reps} pass(es) over {len(sample)} of the {w.rows} rows (every "
                         f"{max(1, w.rows // 64)}th), fp64, in {t_c:.1f}s"}
    out = {
        "metric": "MSA chunked-prefill query rows/s (indexer QK^T on MFMA + per-row top-k + "
                  "sparse attention)",
        "value": w.rows / (ms_step * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.index_k_dtype == 3 else "bf16", "data": "synthetic",
        "config": {"workload": w.name, "recipe": w.recipe, "rows": w.rows,
                   "context_tokens": int(w.seq_lens.sum()), "kv_groups": w.num_groups,
                   "q_heads": w.num_q_heads, "top_k": w.top_k},
        "kernel_us": {"index_contraction": idx_us,
                      "topk_attend_and_gaps": ms_step * 1e3 - idx_us,
                      "sparse_attend": att_us},
        "roofline": {"bound": "mfma", "kernel": "prefill_index_kernel", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "flops_per_launch": flops},
        "cache_write": cw,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
