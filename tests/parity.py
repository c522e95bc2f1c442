"""Helpers shared by the GPU parity tests: device upload of a synthetic
workload, calls through the C ABI, and the comparison rules.

Comparison rules (tolerances of the benchmark spec, made precise):
  * pooled index scores: |S_gpu - S_ref| <= 1e-5 * scale * max_t sum_d |q_d k_td|
    over the block's visible tokens (the standard dot-product error scale);
  * selection: identical sets, except inside a near-tie at the cut, i.e.
    when the oracle's weakest kept and best dropped candidates differ by less
    than 1e-4 relative; then the sets must agree outside the tie band and
    have the same size;
  * attention: max |out_gpu - out_ref| <= 1e-2 (bf16 output vs the fp64
    oracle) for every (row, group): against the oracle's output where the
    selections are identical, against the oracle's attention on the GPU's
    selection where they differ inside the tie band.
"""
from __future__ import annotations

import numpy as np
import torch

import decode_msa_index_amd as msa
import synth
from decode_msa_index_amd import harness

SCORE_RTOL = 1e-5
TIE_RTOL = 1e-4
ATTN_ATOL = 1e-2


def problem(w: synth.Workload, out_dtype=msa.BF16) -> msa.Problem:
    return harness.problem(w, out_dtype)


def oracle_problem(w: synth.Workload, threads: int = 0):
    import oracle
    return oracle.Problem(**w.problem_fields(), num_threads=threads)


def subset_rows(w: synth.Workload, rows) -> synth.Workload:
    """The same caches with only the given query rows of a one-sequence,
    many-row workload: the oracle's share of a sampled comparison."""
    import dataclasses
    assert w.num_seqs == 1 and w.q_pos is not None
    idx = np.asarray(rows, np.int64)
    return dataclasses.replace(
        w, name=w.name + "-sample", rows_per_seq=len(idx),
        index_q=np.ascontiguousarray(w.index_q[idx]), q=np.ascontiguousarray(w.q[idx]),
        q_pos=np.ascontiguousarray(w.q_pos[idx]))


dev = harness.dev
DeviceWorkload = harness.DeviceWorkload


# ---------------------------------------------------------------------------
# independent decoders for the error bound of the scores
# ---------------------------------------------------------------------------

def _f32_of(arr, dtype):
    if dtype == synth.F32:
        return arr.astype(np.float32)
    if dtype == synth.BF16:
        return (arr.astype(np.uint32) << 16).view(np.float32)
    if dtype == synth.FP8:
        return torch.from_numpy(arr).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    raise ValueError(dtype)


_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6], np.float32)


def index_keys_abs(w: synth.Workload, pblocks: np.ndarray) -> np.ndarray:
    """|dequantised index keys| of the given physical blocks, [n, BS, Di] fp32
    (zeros for table entries outside the pool: such a block holds no key)."""
    pblocks = np.asarray(pblocks)
    bad = (pblocks < 0) | (pblocks >= w.num_phys_blocks)
    if bad.any():
        v = index_keys_abs(w, np.where(bad, 0, pblocks))
        v[bad] = 0.0
        return v
    if w.index_k_dtype == synth.NVFP4:
        d = w.ik_data[pblocks]
        s = torch.from_numpy(np.ascontiguousarray(w.ik_scales[pblocks])).view(
            torch.float8_e4m3fn).to(torch.float32).numpy()
        codes = np.stack([d & 15, d >> 4], axis=-1).reshape(d.shape[:-1] + (-1,))
        v = _E2M1[codes] * np.repeat(s, 16, axis=-1)
    else:
        v = _f32_of(w.ik_data[pblocks], w.index_k_dtype)
    return np.abs(v) * np.float32(w.index_k_scale)


def row_pos(w: synth.Workload, r: int) -> int:
    """The last key row r sees: its position clamped to the sequence and to
    the block table's reach (negative: none)."""
    b = r // w.rows_per_seq
    last = min(int(w.seq_lens[b]), w.max_blocks * w.block_size) - 1
    return min(int(w.q_pos[r]), last) if w.q_pos is not None else last


def score_bound(w: synth.Workload) -> np.ndarray:
    """1e-5-relative error bound per (row, group, block)."""
    rows, G, MB, BS = w.rows, w.num_groups, w.max_blocks, w.block_size
    bound = np.zeros((rows, G, MB), np.float32)
    iq = np.abs(_f32_of(w.index_q, w.index_q_dtype))  # [rows, G, Di]
    for r in range(rows):
        b = r // w.rows_per_seq
        pos = row_pos(w, r)
        nb = pos // BS + 1 if pos >= 0 else 0
        for j0 in range(0, nb, 512):
            j1 = min(nb, j0 + 512)
            k = index_keys_abs(w, w.block_table[b, j0:j1])  # [n, BS, Di]
            s = k.reshape(-1, k.shape[-1]) @ iq[r].T  # [n*BS, G]
            s = s.reshape(j1 - j0, BS, G)
            if j1 == nb:
                last = pos - (nb - 1) * BS + 1
                s[-1, last:] = 0.0
            bound[r, :, j0:j1] = s.max(axis=1).T
    return bound * np.float32(SCORE_RTOL * w.index_scale)


def check_scores(w, got: np.ndarray, ref: np.ndarray):
    bound = score_bound(w)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), "-inf pattern differs"
    assert np.all(got[~fin] == ref[~fin])
    err = np.abs(got[fin].astype(np.float64) - ref[fin].astype(np.float64))
    lim = bound[fin].astype(np.float64) + 1e-30
    worst = float(np.max(err / lim)) if err.size else 0.0
    assert worst <= 1.0, f"score error {worst:.3f} x the 1e-5 bound"
    return worst


def selection_matches(w, ref_scores, ref_sel, got_sel, row, g) -> bool:
    """True if identical; raises on an invalid mismatch; False for an allowed
    near-tie difference."""
    a = [int(x) for x in ref_sel[row, g] if x >= 0]
    bsel = [int(x) for x in got_sel[row, g] if x >= 0]
    assert list(got_sel[row, g][len(bsel):]) == [-1] * (w.top_k - len(bsel)), "bad padding"
    assert bsel == sorted(bsel), "selection not ascending"
    if a == bsel:
        return True
    pos = row_pos(w, row)
    rb = pos // w.block_size
    n_local = max(w.local_blocks, 1)
    forced = {j for j in range(rb + 1) if j < w.init_blocks or j > rb - n_local}
    free = [j for j in range(rb + 1) if j not in forced]
    assert forced <= set(bsel) and len(bsel) == len(a), f"row {row} group {g}: {bsel} vs {a}"
    s = ref_scores[row, g].astype(np.float64)
    kept = [j for j in a if j not in forced]
    dropped = [j for j in free if j not in a]
    assert kept and dropped, f"row {row} group {g}: {bsel} vs {a} with nothing to choose"
    cK = min(s[j] for j in kept)
    cK1 = max(s[j] for j in dropped)
    gap = (cK - cK1) / max(abs(cK), 1e-30)
    assert gap < TIE_RTOL, (f"row {row} group {g}: selection differs without a near tie "
                            f"(gap {gap:.2e}): {bsel} vs {a}")
    band = {j for j in free if abs(s[j] - cK) <= TIE_RTOL * abs(cK)}
    assert set(a) - band == set(bsel) - band, f"row {row} group {g}: differs outside the tie band"
    return False


def check_selection(w, ref_scores, ref_sel, got_sel) -> np.ndarray:
    """Returns a bool mask [rows, G] of exact matches."""
    same = np.zeros((w.rows, w.num_groups), bool)
    for r in range(w.rows):
        for g in range(w.num_groups):
            same[r, g] = selection_matches(w, ref_scores, ref_sel, got_sel, r, g)
    return same


def _unit_errors(w, got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Max-abs error per (row, group) unit, [rows, G]."""
    hpg = w.num_q_heads // w.num_groups
    err = np.abs(got.astype(np.float64) - ref)  # [rows, H, D]
    return err.reshape(w.rows, w.num_groups, hpg, -1).max(axis=(2, 3))


def check_attention(w, got: np.ndarray, ref: np.ndarray, atol=ATTN_ATOL):
    """Every (row, group) of the output against the oracle's."""
    err = _unit_errors(w, got, ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, f"attention max-abs error {worst:.3e} > {atol}"
    return worst


def check_decode_attention(w, got: np.ndarray, ref: np.ndarray, same: np.ndarray,
                           got_topk: np.ndarray, atol=ATTN_ATOL):
    """Every (row, group) of a decode output: against the oracle's output
    where the GPU made the oracle's selection, and where the two selections
    differ inside the near-tie band at the cut (both are correct), against the
    oracle's attention recomputed on the GPU's own selection."""
    err = _unit_errors(w, got, ref)
    if not same.all():
        import oracle
        o2, _ = oracle.sparse_attend(oracle_problem(w), w.q, w.kv_data, w.kv_scales,
                                     w.block_table, w.seq_lens,
                                     np.ascontiguousarray(got_topk, np.int32), w.q_pos)
        err = np.where(same, err, _unit_errors(w, got, o2))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, f"attention max-abs error {worst:.3e} > {atol}"
    return worst


# Per-case parity counts, printed in the session summary (tests/conftest.py),
# so that a GPU run's log keeps them: units whose selection is the oracle's,
# units inside the near-tie band, the worst score error as a fraction of its
# bound and the worst attention error (every unit compared).
RECORDS: list[dict] = []


def record(name: str, same: np.ndarray, score_err: float, attn_err: float):
    RECORDS.append({"case": name, "units": int(same.size), "identical": int(same.sum()),
                    "tie_band": int(same.size - same.sum()), "score_err_of_bound": score_err,
                    "attn_max_abs": attn_err})
