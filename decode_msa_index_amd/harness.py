"""Device-side harness over the Python binding: uploads a workload's arrays
(any object with the fields of a generated workload: shapes, dtypes, scales
and numpy arrays) to the GPU, allocates the outputs and workspaces, and calls
the C ABI on them.  Used by the benchmark and the GPU tests; it marshals
arguments only, like the binding itself.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (BF16, OP_ATTEND, OP_DECODE, Problem, block_topk, decode, index_scores,
               new_workspace, sparse_attend)


def problem(w, out_dtype=BF16) -> Problem:
    """The msa_problem of a workload."""
    return Problem(
        num_seqs=w.num_seqs, rows_per_seq=w.rows_per_seq, num_q_heads=w.num_q_heads,
        num_kv_groups=w.num_groups, head_dim=w.head_dim, index_dim=w.index_dim,
        block_size=w.block_size, top_k=w.top_k, max_blocks_per_seq=w.max_blocks,
        num_phys_blocks=w.num_phys_blocks, q_dtype=w.q_dtype, index_q_dtype=w.index_q_dtype,
        kv_dtype=w.kv_dtype, index_k_dtype=w.index_k_dtype, out_dtype=out_dtype,
        sm_scale=w.sm_scale, index_scale=w.index_scale, k_scale=w.k_scale,
        v_scale=w.v_scale, index_k_scale=w.index_k_scale, init_blocks=w.init_blocks,
        local_blocks=w.local_blocks, share_seqs=w.share_seqs)


def dev(a: np.ndarray | None, device="cuda"):
    """A numpy array as a device tensor (bf16 bit patterns travel as int16)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceWorkload:
    """The workload's arrays on the GPU plus output buffers and workspaces."""

    def __init__(self, w, out_dtype=BF16, device="cuda"):
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
        odt = torch.bfloat16 if out_dtype == BF16 else torch.float32
        self.out = torch.empty(rows, H, D, dtype=odt, device=device)
        self.lse = torch.empty(rows, H, dtype=torch.float32, device=device)
        self.ws_attend = new_workspace(self.p, OP_ATTEND, device)
        self.ws_decode = new_workspace(self.p, OP_DECODE, device)

    def copy_with_new_caches(self) -> "DeviceWorkload":
        """The same queries, tables and outputs over fresh copies of the caches
        at other addresses (a model's next layer)."""
        d = DeviceWorkload.__new__(DeviceWorkload)
        d.__dict__.update(self.__dict__)
        d.ik_data = self.ik_data.clone()
        d.kv_data = self.kv_data.clone()
        d.ik_scales = None if self.ik_scales is None else self.ik_scales.clone()
        d.kv_scales = None if self.kv_scales is None else self.kv_scales.clone()
        return d

    def index_scores(self):
        index_scores(self.p, self.index_q, self.ik_data, self.ik_scales, self.block_table,
                     self.seq_lens, self.q_pos, self.scores)

    def block_topk(self, scores=None):
        block_topk(self.p, self.scores if scores is None else scores, self.seq_lens,
                   self.q_pos, self.topk)

    def sparse_attend(self, topk=None):
        sparse_attend(self.p, self.q, self.kv_data, self.kv_scales, self.block_table,
                      self.seq_lens, self.q_pos, self.topk if topk is None else topk,
                      self.out, self.lse, self.ws_attend)

    def chain(self):
        self.index_scores()
        self.block_topk()
        self.sparse_attend()

    def decode(self, with_scores=True):
        decode(self.p, self.index_q, self.ik_data, self.ik_scales, self.q, self.kv_data,
               self.kv_scales, self.block_table, self.seq_lens, self.q_pos,
               self.scores if with_scores else None, self.topk, self.out, self.lse,
               self.ws_decode)
