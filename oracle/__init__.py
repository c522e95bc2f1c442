"""CPU oracle of the MSA decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it,
and nothing here imports the product package: the two sides share only the
input bytes produced by ``synth``.

The arithmetic lives in ``msa_oracle.c`` (plain C, IEEE double); this module
builds it with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmsa_oracle.so")
_SRC = os.path.join(_HERE, "msa_oracle.c")

F32, BF16, FP8, NVFP4 = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math: IEEE double throughout)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
             "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("rows_per_seq", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_groups", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32), ("num_phys_blocks", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("index_q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("index_k_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_double), ("index_scale", ctypes.c_double),
        ("k_scale", ctypes.c_double), ("v_scale", ctypes.c_double),
        ("index_k_scale", ctypes.c_double), ("num_threads", ctypes.c_int32),
        ("init_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        P = ctypes.POINTER(_Problem)
        vp = ctypes.c_void_p
        L.msa_oracle_e4m3.restype = ctypes.c_double
        L.msa_oracle_e4m3.argtypes = [ctypes.c_uint8]
        L.msa_oracle_e2m1.restype = ctypes.c_double
        L.msa_oracle_e2m1.argtypes = [ctypes.c_uint8]
        L.msa_oracle_bf16.restype = ctypes.c_double
        L.msa_oracle_bf16.argtypes = [ctypes.c_uint16]
        L.msa_oracle_index_scores.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.msa_oracle_block_topk.argtypes = [P, vp, vp, vp, vp]
        L.msa_oracle_sparse_attend.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.msa_oracle_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp]
        L.msa_oracle_threads_used.restype = ctypes.c_int
        L.msa_oracle_encode_e4m3.restype = ctypes.c_uint8
        L.msa_oracle_encode_e4m3.argtypes = [ctypes.c_double]
        L.msa_oracle_encode_e2m1.restype = ctypes.c_uint8
        L.msa_oracle_encode_e2m1.argtypes = [ctypes.c_double]
        L.msa_oracle_cache_write.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp]
        _lib = L
    return _lib


@dataclass
class Problem:
    num_seqs: int
    rows_per_seq: int = 1
    num_q_heads: int = 64
    num_groups: int = 4
    head_dim: int = 128
    index_dim: int = 128
    block_size: int = 128
    top_k: int = 16
    max_blocks: int = 1
    num_phys_blocks: int = 1
    q_dtype: int = BF16
    index_q_dtype: int = BF16
    kv_dtype: int = FP8
    index_k_dtype: int = FP8
    sm_scale: float = 128 ** -0.5
    index_scale: float = 128 ** -0.5
    k_scale: float = 1.0
    v_scale: float = 1.0
    index_k_scale: float = 1.0
    num_threads: int = 0
    init_blocks: int = 0
    local_blocks: int = 0

    def c(self) -> _Problem:
        return _Problem(*[getattr(self, f[0]) for f in _Problem._fields_])


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def e4m3(code: int) -> float:
    return lib().msa_oracle_e4m3(code)


def e2m1(nibble: int) -> float:
    return lib().msa_oracle_e2m1(nibble)


def bf16(bits: int) -> float:
    return lib().msa_oracle_bf16(bits)


def _rows(p: Problem) -> int:
    return p.num_seqs * p.rows_per_seq


def index_scores(p: Problem, index_q, ik_data, ik_scales, block_table, seq_lens,
                 q_pos=None) -> np.ndarray:
    out = np.empty((_rows(p), p.num_groups, p.max_blocks), np.float32)
    pc = p.c()
    rc = lib().msa_oracle_index_scores(ctypes.byref(pc), _ptr(index_q), _ptr(ik_data),
                                       _ptr(ik_scales), _ptr(block_table), _ptr(seq_lens),
                                       _ptr(q_pos), _ptr(out))
    if rc:
        raise ValueError("oracle rejected the problem")
    return out


def block_topk(p: Problem, scores, seq_lens, q_pos=None) -> np.ndarray:
    out = np.empty((_rows(p), p.num_groups, p.top_k), np.int32)
    pc = p.c()
    rc = lib().msa_oracle_block_topk(ctypes.byref(pc), _ptr(scores), _ptr(seq_lens),
                                     _ptr(q_pos), _ptr(out))
    if rc:
        raise ValueError("oracle rejected the problem")
    return out


def sparse_attend(p: Problem, q, kv_data, kv_scales, block_table, seq_lens, topk,
                  q_pos=None):
    out = np.empty((_rows(p), p.num_q_heads, p.head_dim), np.float64)
    lse = np.empty((_rows(p), p.num_q_heads), np.float64)
    pc = p.c()
    rc = lib().msa_oracle_sparse_attend(ctypes.byref(pc), _ptr(q), _ptr(kv_data),
                                        _ptr(kv_scales), _ptr(block_table), _ptr(seq_lens),
                                        _ptr(q_pos), _ptr(topk), _ptr(out), _ptr(lse))
    if rc:
        raise ValueError("oracle rejected the problem")
    return out, lse


def decode(p: Problem, index_q, ik_data, ik_scales, q, kv_data, kv_scales,
           block_table, seq_lens, q_pos=None):
    scores = np.empty((_rows(p), p.num_groups, p.max_blocks), np.float32)
    topk = np.empty((_rows(p), p.num_groups, p.top_k), np.int32)
    out = np.empty((_rows(p), p.num_q_heads, p.head_dim), np.float64)
    lse = np.empty((_rows(p), p.num_q_heads), np.float64)
    pc = p.c()
    rc = lib().msa_oracle_decode(ctypes.byref(pc), _ptr(index_q), _ptr(ik_data),
                                 _ptr(ik_scales), _ptr(q), _ptr(kv_data), _ptr(kv_scales),
                                 _ptr(block_table), _ptr(seq_lens), _ptr(q_pos),
                                 _ptr(scores), _ptr(topk), _ptr(out), _ptr(lse))
    if rc:
        raise ValueError("oracle rejected the problem")
    return scores, topk, out, lse


def threads_used() -> int:
    return lib().msa_oracle_threads_used()


def encode_e4m3(x: float) -> int:
    return lib().msa_oracle_encode_e4m3(x)


def encode_e2m1(x: float) -> int:
    return lib().msa_oracle_encode_e2m1(x)


def cache_write(p: Problem, token_seq, token_pos, k_new, v_new, ik_new, block_table,
                kv_data, kv_scales, ik_data, ik_scales) -> None:
    """Quantises the new tokens into the caches, in place (the arrays are
    updated)."""
    pc = p.c()
    rc = lib().msa_oracle_cache_write(ctypes.byref(pc), len(token_seq), _ptr(token_seq),
                                      _ptr(token_pos), _ptr(k_new), _ptr(v_new), _ptr(ik_new),
                                      _ptr(block_table), _ptr(kv_data), _ptr(kv_scales),
                                      _ptr(ik_data), _ptr(ik_scales))
    if rc:
        raise ValueError("oracle rejected the problem")
