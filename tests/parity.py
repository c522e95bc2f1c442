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
    oracle), checked for every (row, group) whose selection equals the
    oracle's.
"""
from __future__ import annotations

import numpy as np
import torch

import decode_msa_index_amd as msa
import synth

SCORE_RTOL = 1e-5
TIE_RTOL = 1e-4
ATTN_ATOL = 1e-2


def problem(w: synth.Workload, out_dtype=msa.BF16) -> msa.Problem:
    return msa.Problem(
        num_seqs=w.num_seqs, rows_per_seq=w.rows_per_seq, num_q_heads=w.num_q_heads,
        num_kv_groups=w.num_groups, head_dim=w.head_dim, index_dim=w.index_dim,
        block_size=w.block_size, top_k=w.top_k, max_blocks_per_seq=w.max_blocks,
        num_phys_blocks=w.num_phys_blocks, q_dtype=w.q_dtype, index_q_dtype=w.index_q_dtype,
        kv_dtype=w.kv_dtype, index_k_dtype=w.index_k_dtype, out_dtype=out_dtype,
        sm_scale=w.sm_scale, index_scale=w.index_scale, k_scale=w.k_scale,
        v_scale=w.v_scale, index_k_scale=w.index_k_scale, init_blocks=w.init_blocks,
        local_blocks=w.local_blocks, share_seqs=w.share_seqs)


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


def dev(a: np.ndarray | None, device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceWorkload:
    """The workload's arrays on the GPU plus output buffers."""

    def __init__(self, w: synth.Workload, out_dtype=msa.BF16, device="cuda"):
        self.w = w
        self.p = problem(w, out_dtype)
        self.index_q = dev(w.index_q, device)
        self.q = dev(w.q, device)
        self.ik_data = dev(w.ik_data, device)
        self.ik_scales = dev(w.ik_scales, device)
        self.kv_data = dev(w.kv_data, device)
        self.kv_scales = dev(w.kv_scales, device)
        self.block_table = dev(w.block_table, device)
        self.seq_lens = dev(w.seq_lens, device)
        self.q_pos = dev(w.q_pos, device)
        rows, G, H, D = w.rows, w.num_groups, w.num_q_heads, w.head_dim
        self.scores = torch.empty(rows, G, w.max_blocks, dtype=torch.float32, device=device)
        self.topk = torch.empty(rows, G, w.top_k, dtype=torch.int32, device=device)
        odt = torch.bfloat16 if out_dtype == msa.BF16 else torch.float32
        self.out = torch.empty(rows, H, D, dtype=odt, device=device)
        self.lse = torch.empty(rows, H, dtype=torch.float32, device=device)
        self.ws_attend = msa.new_workspace(self.p, msa.OP_ATTEND, device)
        self.ws_decode = msa.new_workspace(self.p, msa.OP_DECODE, device)

    def index_scores(self):
        msa.index_scores(self.p, self.index_q, self.ik_data, self.ik_scales, self.block_table,
                         self.seq_lens, self.q_pos, self.scores)

    def block_topk(self, scores=None):
        msa.block_topk(self.p, self.scores if scores is None else scores, self.seq_lens,
                       self.q_pos, self.topk)

    def sparse_attend(self, topk=None):
        msa.sparse_attend(self.p, self.q, self.kv_data, self.kv_scales, self.block_table,
                          self.seq_lens, self.q_pos, self.topk if topk is None else topk,
                          self.out, self.lse, self.ws_attend)

    def chain(self):
        self.index_scores()
        self.block_topk()
        self.sparse_attend()

    def decode(self, with_scores=True):
        msa.decode(self.p, self.index_q, self.ik_data, self.ik_scales, self.q, self.kv_data,
                   self.kv_scales, self.block_table, self.seq_lens, self.q_pos,
                   self.scores if with_scores else None, self.topk, self.out, self.lse,
                   self.ws_decode)


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
    """|dequantised index keys| of the given physical blocks, [n, BS, Di] fp32."""
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


def check_attention(w, got: np.ndarray, ref: np.ndarray, mask=None, atol=ATTN_ATOL):
    hpg = w.num_q_heads // w.num_groups
    err = np.abs(got.astype(np.float64) - ref)  # [rows, H, D]
    err = err.reshape(w.rows, w.num_groups, hpg, -1).max(axis=(2, 3))
    if mask is not None:
        err = np.where(mask, err, 0.0)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, f"attention max-abs error {worst:.3e} > {atol}"
    return worst
