"""MI355X (gfx950) MiniMax Sparse Attention decode path -- Python binding.

A thin ctypes layer over ``libmsa.so`` (the C ABI in ``include/msa.h``).  It
only marshals arguments: tensors become device pointers, ``None`` becomes
NULL, the stream defaults to torch's current stream.  Every step of the path
runs in the library's HIP kernels; there is no other implementation here, and
importing this package fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

F32, BF16, FP8_E4M3, NVFP4 = 0, 1, 2, 3
OP_INDEX, OP_TOPK, OP_ATTEND, OP_DECODE, OP_CACHE_WRITE = 0, 1, 2, 3, 4

STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARGUMENT", 2: "MSA_ERR_UNSUPPORTED",
          3: "MSA_ERR_WORKSPACE_TOO_SMALL", 4: "MSA_ERR_HIP", 5: "MSA_ERR_DEVICE_WAIT"}

EXPORTS = ["msa_check_problem", "msa_workspace_bytes", "msa_index_scores", "msa_block_topk",
           "msa_sparse_attend", "msa_decode", "msa_decode_static", "msa_cache_write",
           "msa_workspace_status",
           "msa_set_merge_spin_limit", "msa_status_string", "msa_last_error"]


class MsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class MsaProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("rows_per_seq", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_groups", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("num_phys_blocks", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("index_q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("index_k_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("index_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("index_k_scale", ctypes.c_float),
        ("init_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
        ("share_seqs", ctypes.c_int32),
    ]


@dataclass
class Problem:
    """Host description of one call (mirrors ``msa_problem``)."""
    num_seqs: int
    rows_per_seq: int = 1
    num_q_heads: int = 64
    num_kv_groups: int = 4
    head_dim: int = 128
    index_dim: int = 128
    block_size: int = 128
    top_k: int = 16
    max_blocks_per_seq: int = 1
    num_phys_blocks: int = 1
    q_dtype: int = BF16
    index_q_dtype: int = BF16
    kv_dtype: int = FP8_E4M3
    index_k_dtype: int = FP8_E4M3
    out_dtype: int = BF16
    sm_scale: float = 128 ** -0.5
    index_scale: float = 128 ** -0.5
    k_scale: float = 1.0
    v_scale: float = 1.0
    index_k_scale: float = 1.0
    init_blocks: int = 0
    local_blocks: int = 0
    share_seqs: int = 0

    def c(self) -> MsaProblem:
        return MsaProblem(*[getattr(self, f.name) for f in fields(self)])


_lib = None


def lib():
    """Load libmsa.so; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run decode_msa_index_amd/build.py "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(MsaProblem)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.msa_check_problem.restype = ctypes.c_int
        L.msa_check_problem.argtypes = [P, i32]
        L.msa_workspace_bytes.restype = ctypes.c_int
        L.msa_workspace_bytes.argtypes = [P, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.msa_index_scores.restype = ctypes.c_int
        L.msa_index_scores.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.msa_block_topk.restype = ctypes.c_int
        L.msa_block_topk.argtypes = [P, vp, vp, vp, vp, vp]
        L.msa_sparse_attend.restype = ctypes.c_int
        L.msa_sparse_attend.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        ctypes.c_size_t, vp]
        L.msa_decode.restype = ctypes.c_int
        L.msa_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 ctypes.c_size_t, vp]
        L.msa_decode_static.restype = ctypes.c_int
        L.msa_decode_static.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp]
        L.msa_cache_write.restype = ctypes.c_int
        L.msa_cache_write.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.msa_workspace_status.restype = ctypes.c_int
        L.msa_workspace_status.argtypes = [vp, vp]
        L.msa_set_merge_spin_limit.restype = None
        L.msa_set_merge_spin_limit.argtypes = [i32]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_last_error.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != 0:
        raise MsaError(rc, lib().msa_last_error().decode())


def check_problem(p: Problem, op: int) -> int:
    """Host validation only (no HIP call); returns the status code."""
    pc = p.c()
    return lib().msa_check_problem(ctypes.byref(pc), op)


def workspace_bytes(p: Problem, op: int) -> int:
    pc = p.c()
    out = ctypes.c_size_t(0)
    _check(lib().msa_workspace_bytes(ctypes.byref(pc), op, ctypes.byref(out)))
    return out.value


def index_scores(p: Problem, index_q, ik_data, ik_scales, block_table, seq_lens, q_pos,
                 block_scores, stream=None):
    pc = p.c()
    _check(lib().msa_index_scores(ctypes.byref(pc), _ptr(index_q), _ptr(ik_data),
                                  _ptr(ik_scales), _ptr(block_table), _ptr(seq_lens),
                                  _ptr(q_pos), _ptr(block_scores), _stream(stream)))


def block_topk(p: Problem, block_scores, seq_lens, q_pos, topk_idx, stream=None):
    pc = p.c()
    _check(lib().msa_block_topk(ctypes.byref(pc), _ptr(block_scores), _ptr(seq_lens),
                                _ptr(q_pos), _ptr(topk_idx), _stream(stream)))


def sparse_attend(p: Problem, q, kv_data, kv_scales, block_table, seq_lens, q_pos, topk_idx,
                  out, lse, workspace, stream=None):
    pc = p.c()
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().msa_sparse_attend(ctypes.byref(pc), _ptr(q), _ptr(kv_data), _ptr(kv_scales),
                                   _ptr(block_table), _ptr(seq_lens), _ptr(q_pos),
                                   _ptr(topk_idx), _ptr(out), _ptr(lse), _ptr(workspace),
                                   nbytes, _stream(stream)))


def decode(p: Problem, index_q, ik_data, ik_scales, q, kv_data, kv_scales, block_table,
           seq_lens, q_pos, block_scores, topk_idx, out, lse, workspace, stream=None):
    pc = p.c()
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().msa_decode(ctypes.byref(pc), _ptr(index_q), _ptr(ik_data), _ptr(ik_scales),
                            _ptr(q), _ptr(kv_data), _ptr(kv_scales), _ptr(block_table),
                            _ptr(seq_lens), _ptr(q_pos), _ptr(block_scores), _ptr(topk_idx),
                            _ptr(out), _ptr(lse), _ptr(workspace), nbytes, _stream(stream)))


def decode_static(p: Problem, index_q, ik_data, ik_scales, q, kv_data, kv_scales, block_table,
                  seq_lens, q_pos, block_scores, topk_idx, out, lse, stream=None):
    """msa_decode on the library's own static scratch (no workspace)."""
    pc = p.c()
    _check(lib().msa_decode_static(ctypes.byref(pc), _ptr(index_q), _ptr(ik_data),
                                   _ptr(ik_scales), _ptr(q), _ptr(kv_data), _ptr(kv_scales),
                                   _ptr(block_table), _ptr(seq_lens), _ptr(q_pos),
                                   _ptr(block_scores), _ptr(topk_idx), _ptr(out), _ptr(lse),
                                   _stream(stream)))


def cache_write(p: Problem, token_seq, token_pos, k_new, v_new, ik_new, block_table, kv_data,
                kv_scales, ik_data, ik_scales, stream=None):
    """Quantise new tokens into the caches (in place)."""
    pc = p.c()
    n = int(token_seq.numel()) if token_seq is not None else 0
    _check(lib().msa_cache_write(ctypes.byref(pc), n, _ptr(token_seq), _ptr(token_pos),
                                 _ptr(k_new), _ptr(v_new), _ptr(ik_new), _ptr(block_table),
                                 _ptr(kv_data), _ptr(kv_scales), _ptr(ik_data),
                                 _ptr(ik_scales), _stream(stream)))


def workspace_status(workspace, stream=None) -> int:
    """Waits for the stream and returns the workspace's status code (0, or
    5 = MSA_ERR_DEVICE_WAIT after a split-K merge gave up); raises on other
    errors."""
    rc = lib().msa_workspace_status(_ptr(workspace), _stream(stream))
    if rc not in (0, 5):
        _check(rc)
    return rc


def set_merge_spin_limit(polls: int) -> None:
    """Test hook: polls before a split-K merge gives up (negative: at once)."""
    lib().msa_set_merge_spin_limit(polls)


def new_workspace(p: Problem, op: int, device="cuda"):
    """A zero-filled workspace of the size the call needs (torch allocation)."""
    import torch
    n = max(workspace_bytes(p, op), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)
