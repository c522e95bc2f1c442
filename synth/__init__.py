"""Seeded synthetic workloads for the MSA decode path.

Both the CPU oracle and the HIP library consume the bytes made here.  This
module holds none of the method's arithmetic: it draws counter-based normals
(``synth.c``), encodes them into the stored formats (bf16, OCP e4m3fn,
NVFP4), and lays out the paged caches, block tables and lengths.

Workload recipes (shapes of the pages' workloads; all values seeded):

* ``tiny``    1 sequence of 4,096 tokens (32 blocks), 4 groups x 4 heads,
              fp32 everything, identity block table, +2.0 added to every
              index-key element of 3 random blocks.
* ``fp8_b32`` 32 sequences x 32,768 tokens, 64 query heads in 4 groups,
              bf16 queries, e4m3 K/V/index keys (tensor scales 1.0), random
              permutation block table.
* ``fp8_long`` 8 sequences, lengths uniform in [131,072, 262,144] (a partial
              last block allowed), as ``fp8_b32`` plus 8 planted high-score
              blocks per sequence.
* ``nvfp4_512k`` 4 sequences x 524,288 tokens, NVFP4 K/V/index keys.
* ``custom``  any of the above knobs, for edge cases.

Layouts are documented in ``include/msa.h``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmsa_synth.so")
_SRC = os.path.join(_HERE, "synth.c")

F32, BF16, FP8, NVFP4 = 0, 1, 2, 3
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3", NVFP4: "nvfp4"}

# NVFP4 per-tensor scale used by the quantiser: values of magnitude up to 8
# map onto the largest e4m3 scale (448) times the largest E2M1 value (6).
NVFP4_TENSOR_SCALE = 8.0 / (6.0 * 448.0)

STREAM_INDEX_Q, STREAM_Q, STREAM_IK, STREAM_KV = 1, 2, 3, 4
STREAM_TABLE, STREAM_LENS, STREAM_PLANT = 5, 6, 7
STREAM_SHARED_Q = 8


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-std=gnu11", "-fPIC", "-shared",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        u64, vp = ctypes.c_uint64, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        L.synth_u64.argtypes = [u64, u64, u64, vp]
        L.synth_normal_f32.argtypes = [u64, u64, u64, vp]
        L.synth_normal_e4m3.argtypes = [u64, u64, u64, vp]
        L.synth_encode_e4m3.argtypes = [vp, u64, vp]
        L.synth_encode_bf16.argtypes = [vp, u64, vp]
        L.synth_nvfp4_rows.argtypes = [vp, u64, ctypes.c_int, ctypes.c_float, vp, vp]
        i32, f32 = ctypes.c_int, ctypes.c_float
        L.synth_kv_fp8.argtypes = [u64, u64, u64, i32, i32, i32, vp]
        L.synth_kv_nvfp4.argtypes = [u64, u64, u64, i32, i32, i32, f32, vp, vp]
        L.synth_ik.argtypes = [u64, u64, u64, i32, i32, i32, f32, vp, vp]
        _lib = L
    return _lib


def key(seed: int, stream: int) -> int:
    return lib().synth_key(seed, stream)


def normal(seed: int, stream: int, first: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(key(seed, stream), first, n, out.ctypes.data)
    return out


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().synth_encode_e4m3(x.ctypes.data, x.size, out.ctypes.data)
    return out


def encode_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().synth_encode_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def encode_nvfp4_rows(x: np.ndarray, g: float = NVFP4_TENSOR_SCALE):
    """x[..., dim] -> (data[..., dim/2], scales[..., dim/16])."""
    x = np.ascontiguousarray(x, np.float32)
    dim = x.shape[-1]
    rows = x.size // dim
    data = np.empty(x.shape[:-1] + (dim // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (dim // 16,), np.uint8)
    lib().synth_nvfp4_rows(x.ctypes.data, rows, dim, g, data.ctypes.data,
                           scales.ctypes.data)
    return data, scales


def _nibbles_T(data: np.ndarray) -> np.ndarray:
    """[..., t, d/2] packed along d -> [..., d, t/2] packed along t."""
    lo = data & 15
    hi = data >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(data.shape[:-1] + (data.shape[-1] * 2,))
    codes = np.swapaxes(codes, -1, -2)  # [..., d, t]
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass
class Workload:
    name: str
    num_seqs: int
    rows_per_seq: int
    num_q_heads: int
    num_groups: int
    head_dim: int
    index_dim: int
    block_size: int
    top_k: int
    max_blocks: int
    num_phys_blocks: int
    q_dtype: int
    index_q_dtype: int
    kv_dtype: int
    index_k_dtype: int
    sm_scale: float
    index_scale: float
    k_scale: float
    v_scale: float
    index_k_scale: float
    index_q: np.ndarray
    q: np.ndarray
    ik_data: np.ndarray
    ik_scales: np.ndarray | None
    kv_data: np.ndarray
    kv_scales: np.ndarray | None
    block_table: np.ndarray
    seq_lens: np.ndarray
    q_pos: np.ndarray | None
    planted: dict = field(default_factory=dict)
    init_blocks: int = 0    # leading blocks always selected
    local_blocks: int = 0   # trailing blocks always selected (0, 1: the recent one)
    share_seqs: int = 0     # share groups of the index scan (a hint to the kernels only)
    recipe: str = ""

    @property
    def rows(self) -> int:
        return self.num_seqs * self.rows_per_seq

    def problem_fields(self) -> dict:
        keys = ["num_seqs", "rows_per_seq", "num_q_heads", "num_groups", "head_dim",
                "index_dim", "block_size", "top_k", "max_blocks", "num_phys_blocks",
                "q_dtype", "index_q_dtype", "kv_dtype", "index_k_dtype", "sm_scale",
                "index_scale", "k_scale", "v_scale", "index_k_scale", "init_blocks",
                "local_blocks"]
        return {k: getattr(self, k) for k in keys}

    def index_tokens(self) -> int:
        if self.q_pos is not None:
            return int(np.sum(self.q_pos.astype(np.int64) + 1))
        return int(np.sum(self.seq_lens.astype(np.int64)))


def _encode_plain(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x, np.float32)
    if dtype == BF16:
        return encode_bf16(x)
    if dtype == FP8:
        return encode_e4m3(x)
    raise ValueError(dtype)


def _bytes_per(dtype: int) -> int:
    return {F32: 4, BF16: 2, FP8: 1}[dtype]


def make(name: str = "custom", *, seed: int = 0x4D5341, seq_lens=None, num_seqs: int = 1,
         rows_per_seq: int = 1, q_pos=None, num_q_heads: int = 64, num_groups: int = 4,
         head_dim: int = 128, index_dim: int = 128, block_size: int = 128, top_k: int = 16,
         q_dtype: int = BF16, index_q_dtype: int | None = None, kv_dtype: int = FP8,
         index_k_dtype: int | None = None, table: str = "permute", extra_phys: int = 0,
         plant_per_seq: int = 0, plant_add: float = 1.0, bump_blocks: int = 0,
         bump_add: float = 2.0, max_blocks: int | None = None, k_scale: float = 1.0,
         v_scale: float = 1.0, ik_scale: float | None = None,
         kv_fill: bool = True, share_seqs: int = 0, share_blocks: int = 0,
         share_corr: float = 0.0) -> Workload:
    """Build one seeded workload.

    table: "identity" (seq b's block j is physical b*max_blocks+j) or
    "permute" (a seeded random permutation of the physical pool).
    plant_per_seq: add ``plant_add * sign(sum_g index_q[b, g, :])`` to every
    index-key element of that many random non-recent blocks per sequence.
    bump_blocks: add ``bump_add`` to every index-key element of that many
    random blocks (of sequence 0).
    kv_fill: False leaves the K/V pool zero (timing-only callers).
    share_seqs, share_blocks: consecutive groups of share_seqs sequences
    (requests with a common prefix) map their first logical blocks -- up to
    share_blocks, and short of every member's last block -- to the same
    physical blocks ("permute" tables only); share_seqs is also passed to the
    kernels as the share-group hint.
    share_corr: rho in [0, 1) for groups with a shared prefix: every member's
    queries and index queries become rho * (the group's common draw) +
    sqrt(1 - rho^2) * (its own draw) -- requests continuing one prompt -- and
    plant_per_seq blocks are planted once per group, inside the shared
    prefix, along the common index query's direction instead of per member.
    """
    index_q_dtype = q_dtype if index_q_dtype is None else index_q_dtype
    index_k_dtype = kv_dtype if index_k_dtype is None else index_k_dtype
    seq_lens = np.asarray(seq_lens if seq_lens is not None else [4096] * num_seqs,
                          dtype=np.int64)
    num_seqs = len(seq_lens)
    BS = block_size
    nb = (seq_lens + BS - 1) // BS
    if max_blocks is None:
        max_blocks = int(max(1, nb.max() if num_seqs else 1))
    rows = num_seqs * rows_per_seq
    G, H, D, Di = num_groups, num_q_heads, head_dim, index_dim

    # ---- block table ----
    groups = []  # (first sequence, end, shared blocks)
    if share_seqs > 1 and share_blocks > 0:
        if table != "permute":
            raise ValueError("shared prefixes need a permuted table")
        for g0 in range(0, num_seqs, share_seqs):
            g1 = min(num_seqs, g0 + share_seqs)
            groups.append((g0, g1, int(min(share_blocks, int(nb[g0:g1].min()) - 1))))
    else:
        groups = [(b, b + 1, 0) for b in range(num_seqs)]
    P = int(nb.sum()) - sum((g1 - g0 - 1) * sh for g0, g1, sh in groups) + extra_phys
    P = max(P, 1)
    bt = np.zeros((num_seqs, max_blocks), np.int32)
    if table == "identity":
        P = max(P, num_seqs * max_blocks)
        for b in range(num_seqs):
            bt[b, : nb[b]] = np.arange(b * max_blocks, b * max_blocks + nb[b])
    else:
        perm = np.random.default_rng([seed, STREAM_TABLE]).permutation(P).astype(np.int32)
        off = 0
        for g0, g1, sh in groups:
            shared = perm[off: off + sh]
            off += sh
            for b in range(g0, g1):
                bt[b, :sh] = shared
                bt[b, sh: nb[b]] = perm[off: off + nb[b] - sh]
                off += nb[b] - sh

    # ---- queries ----
    iq_f = normal(seed, STREAM_INDEX_Q, 0, rows * G * Di).reshape(rows, G, Di)
    q_f = normal(seed, STREAM_Q, 0, rows * H * D).reshape(rows, H, D)
    corr_groups = [(g0, g1, sh) for g0, g1, sh in groups if g1 - g0 > 1 and sh > 0] \
        if share_corr > 0 else []
    if corr_groups:
        if rows_per_seq != 1:
            raise ValueError("share_corr needs rows_per_seq == 1")
        rho = float(share_corr)
        own = math.sqrt(1.0 - rho * rho)
        per = G * Di + H * D
        for n, (g0, g1, _) in enumerate(corr_groups):
            c = normal(seed, STREAM_SHARED_Q, n * per, per)
            iq_f[g0:g1] = rho * c[:G * Di].reshape(1, G, Di) + own * iq_f[g0:g1]
            q_f[g0:g1] = rho * c[G * Di:].reshape(1, H, D) + own * q_f[g0:g1]
    index_q = _encode_plain(iq_f, index_q_dtype)
    q = _encode_plain(q_f, q_dtype)

    # ---- planted / bumped index-key blocks (added before encoding) ----
    add_vec = {}  # physical block -> vector added to every token of the block
    planted = {}
    rng_p = np.random.default_rng([seed, STREAM_PLANT])
    if plant_per_seq:
        iq_vals = (index_q.astype(np.uint32) << 16).view(np.float32) \
            if index_q_dtype == BF16 else index_q.astype(np.float32)
        in_corr = set()
        for g0, g1, sh in corr_groups:  # once per group, inside the shared prefix
            in_corr.update(range(g0, g1))
            choices = rng_p.choice(sh, size=min(plant_per_seq, sh), replace=False)
            js = sorted(int(c) for c in choices)
            u = np.sign(iq_vals[g0 * rows_per_seq:g1 * rows_per_seq].astype(np.float64)
                        .sum(axis=(0, 1))).astype(np.float32)
            u[u == 0] = 1.0
            for b in range(g0, g1):
                planted[b] = js
            for j in js:
                add_vec[int(bt[g0, j])] = plant_add * u
        for b in range(num_seqs):
            if b in in_corr:
                continue
            recent = int(nb[b]) - 1
            choices = rng_p.choice(recent, size=min(plant_per_seq, recent), replace=False)
            planted[b] = sorted(int(c) for c in choices)
            r0 = b * rows_per_seq
            u = np.sign(iq_vals[r0].astype(np.float64).sum(axis=0)).astype(np.float32)
            u[u == 0] = 1.0
            for j in planted[b]:
                add_vec[int(bt[b, j])] = plant_add * u
    if bump_blocks:
        choices = rng_p.choice(int(nb[0]), size=min(bump_blocks, int(nb[0])), replace=False)
        planted[0] = sorted(int(c) for c in choices)
        for j in planted[0]:
            add_vec[int(bt[0, j])] = np.full(Di, bump_add, np.float32)

    # ---- index-key pool ----
    ik_scales = None
    if index_k_dtype == NVFP4:
        ik_data = np.empty((P, BS, Di // 2), np.uint8)
        ik_scales = np.empty((P, BS, Di // 16), np.uint8)
    else:
        ik_data = np.empty((P, BS, Di), np.float32 if index_k_dtype == F32 else np.uint8)
    per_blk = BS * Di
    chunk = max(1, (1 << 22) // per_blk)

    def gen_ik(p0):
        p1 = min(P, p0 + chunk)
        if index_k_dtype in (FP8, NVFP4):
            sc_ptr = ik_scales[p0:p1].ctypes.data if ik_scales is not None else None
            lib().synth_ik(key(seed, STREAM_IK), p0, p1 - p0, BS, Di, index_k_dtype,
                           NVFP4_TENSOR_SCALE, ik_data[p0:p1].ctypes.data, sc_ptr)
            return
        x = normal(seed, STREAM_IK, p0 * per_blk, (p1 - p0) * per_blk).reshape(p1 - p0, BS, Di)
        ik_data[p0:p1] = _encode_plain(x, index_k_dtype)

    def plant_ik(pb):
        x = normal(seed, STREAM_IK, pb * per_blk, per_blk).reshape(BS, Di)
        x += add_vec[pb][None, :]
        if index_k_dtype == NVFP4:
            d, s_ = encode_nvfp4_rows(x)
            ik_data[pb] = d
            ik_scales[pb] = s_
        else:
            ik_data[pb] = _encode_plain(x, index_k_dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(gen_ik, range(0, P, chunk)))
        list(ex.map(plant_ik, sorted(add_vec)))

    # ---- K/V pool: plane 0 = K [t][d], plane 1 = V^T [d][t] ----
    kv_scales = None
    per_kv = 2 * G * BS * D
    if kv_dtype == NVFP4:
        kv_data = np.zeros((P, 2, G, BS * D // 2), np.uint8)
        kv_scales = np.zeros((P, 2, G, BS * D // 16), np.uint8)
    elif kv_dtype == F32:
        kv_data = np.zeros((P, 2, G, BS, D), np.float32)
    else:
        kv_data = np.zeros((P, 2, G, BS, D), np.uint8)
    chunk_kv = max(1, (1 << 22) // per_kv)

    def gen_kv(p0):
        p1 = min(P, p0 + chunk_kv)
        if kv_dtype == NVFP4:
            lib().synth_kv_nvfp4(key(seed, STREAM_KV), p0, p1 - p0, G, BS, D,
                                 NVFP4_TENSOR_SCALE, kv_data[p0:p1].ctypes.data,
                                 kv_scales[p0:p1].ctypes.data)
        elif kv_dtype == FP8:
            lib().synth_kv_fp8(key(seed, STREAM_KV), p0, p1 - p0, G, BS, D,
                               kv_data[p0:p1].ctypes.data)
        else:
            x = normal(seed, STREAM_KV, p0 * per_kv, (p1 - p0) * per_kv).reshape(
                p1 - p0, 2, G, BS, D)
            x[:, 1] = np.swapaxes(x[:, 1], -1, -2)
            kv_data[p0:p1] = x

    if kv_fill:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(gen_kv, range(0, P, chunk_kv)))

    if ik_scale is None:
        ik_scale = NVFP4_TENSOR_SCALE if index_k_dtype == NVFP4 else 1.0
    if kv_dtype == NVFP4:
        k_scale = k_scale * NVFP4_TENSOR_SCALE
        v_scale = v_scale * NVFP4_TENSOR_SCALE
    qp = None if q_pos is None else np.ascontiguousarray(q_pos, np.int32)
    return Workload(
        name=name, num_seqs=num_seqs, rows_per_seq=rows_per_seq, num_q_heads=H,
        num_groups=G, head_dim=D, index_dim=Di, block_size=BS, top_k=top_k,
        max_blocks=max_blocks, num_phys_blocks=P, q_dtype=q_dtype,
        index_q_dtype=index_q_dtype, kv_dtype=kv_dtype, index_k_dtype=index_k_dtype,
        sm_scale=D ** -0.5, index_scale=Di ** -0.5, k_scale=k_scale, v_scale=v_scale,
        index_k_scale=ik_scale, index_q=index_q, q=q, ik_data=ik_data,
        ik_scales=ik_scales, kv_data=kv_data, kv_scales=kv_scales, block_table=bt,
        seq_lens=seq_lens.astype(np.int32), q_pos=qp, planted=planted,
        share_seqs=share_seqs)


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------

def tiny(seed: int = 0x4D5341 + 1) -> Workload:
    w = make("tiny", seed=seed, seq_lens=[4096], num_q_heads=16, num_groups=4,
             q_dtype=F32, kv_dtype=F32, table="identity", bump_blocks=3, bump_add=2.0)
    w.recipe = ("1 seq x 4096 tokens, 4 groups x 4 heads, D=Di=128, fp32, N(0,1), "
                "+2.0 on all index-key elements of 3 random blocks, identity table")
    return w


def fp8_b32(seed: int = 0x4D5341 + 2, **kw) -> Workload:
    w = make("fp8_b32", seed=seed, seq_lens=[32768] * 32, q_dtype=BF16, kv_dtype=FP8, **kw)
    w.recipe = ("32 seqs x 32768 tokens, 64 q heads / 4 groups, D=Di=128, bf16 q, "
                "e4m3 K/V/index keys (scale 1.0), N(0,1), random permutation table")
    return w


def long_lens(seed: int, n: int = 8, lo: int = 131072, hi: int = 262144) -> np.ndarray:
    rng = np.random.default_rng([seed, STREAM_LENS])
    return rng.integers(lo, hi + 1, size=n).astype(np.int64)


def fp8_long(seed: int = 0x4D5341 + 3, **kw) -> Workload:
    w = make("fp8_long", seed=seed, seq_lens=long_lens(seed), q_dtype=BF16,
             kv_dtype=FP8, plant_per_seq=8, plant_add=1.0, **kw)
    w.recipe = ("8 seqs, lengths U[131072, 262144], 64 q heads / 4 groups, D=Di=128, "
                "bf16 q, e4m3 K/V/index keys, N(0,1), 8 planted blocks per seq "
                "(+1.0*sign(sum_g qI) before rounding), random permutation table")
    return w


def fp8_256k(seed: int = 0x4D5341 + 5, **kw) -> Workload:
    w = make("fp8_256k", seed=seed, seq_lens=[262144] * 8, q_dtype=BF16, kv_dtype=FP8,
             plant_per_seq=8, plant_add=1.0, **kw)
    w.recipe = ("8 seqs x 262144 tokens (256K, batch 8), 64 q heads / 4 groups, D=Di=128, "
                "bf16 q, e4m3 K/V/index keys, N(0,1), 8 planted blocks per seq "
                "(+1.0*sign(sum_g qI) before rounding), random permutation table")
    return w


def _share64(name: str, kv_dtype: int, seed: int, **kw) -> Workload:
    """64 requests with a common 128K-token prefix (the same physical blocks
    in every block table) and private continuations of U[1, 8192] tokens,
    declared as one share group of 64."""
    pre = 131072
    rng = np.random.default_rng([seed, STREAM_TABLE, 1])
    lens = (pre + rng.integers(1, 8193, size=64)).tolist()
    w = make(name, seed=seed, seq_lens=lens, q_dtype=BF16, kv_dtype=kv_dtype,
             plant_per_seq=8, plant_add=1.0, share_seqs=64, share_blocks=pre // 128, **kw)
    fmt = "e4m3 K/V/index keys, N(0,1)" if kv_dtype == FP8 else \
        "NVFP4 K/V/index keys quantised from N(0,1)"
    w.recipe = ("64 requests sharing a 131072-token prefix (same physical blocks) plus "
                "U[1, 8192] private tokens each, one share group of 64, 64 q heads / 4 "
                f"groups, D=Di=128, bf16 q, {fmt}, 8 planted blocks "
                "per request, random permutation table")
    return w


def fp8_share64(seed: int = 0x4D5341 + 9, **kw) -> Workload:
    return _share64("fp8_share64", FP8, seed, **kw)


def nvfp4_share64(seed: int = 0x4D5341 + 11, **kw) -> Workload:
    """The shared-prefix batch with NVFP4 K/V and index keys."""
    return _share64("nvfp4_share64", NVFP4, seed, **kw)


def fp8_dcp45_shard(seed: int = 0x4D5341 + 10, **kw) -> Workload:
    """One GPU's share of a context-parallel (DCP, 4 GPUs) indexer step over
    45 requests of U[30,720, 215,040] tokens: each GPU scores a quarter of
    every request's context for all 4 index heads."""
    rng = np.random.default_rng([seed, STREAM_TABLE, 2])
    full = rng.integers(30720, 215041, size=45)
    lens = ((full + 3) // 4).tolist()
    w = make("fp8_dcp45_shard", seed=seed, seq_lens=lens, q_dtype=BF16, kv_dtype=FP8,
             plant_per_seq=8, plant_add=1.0, **kw)
    w.recipe = ("one GPU's quarter of a 4-way context-parallel step: 45 requests, each a "
                "quarter of U[30720, 215040] tokens, 64 q heads / 4 groups, D=Di=128, bf16 q, "
                "e4m3 K/V/index keys, N(0,1), 8 planted blocks per request, random "
                "permutation table")
    return w


def spec4_256k(seed: int = 0x4D5341 + 7, **kw) -> Workload:
    """Speculative decode: the 256K batch-8 caches with 4 query rows per
    sequence at its last 4 positions (each row its own causal end)."""
    L, R = 262144, 4
    qp = np.concatenate([np.arange(L - R, L)] * 8).astype(np.int32)
    w = make("spec4_256k", seed=seed, seq_lens=[L] * 8, rows_per_seq=R, q_pos=qp,
             q_dtype=BF16, kv_dtype=FP8, plant_per_seq=8, plant_add=1.0, **kw)
    w.recipe = ("8 seqs x 262144 tokens, 4 speculative query rows per seq at positions "
                "262140..262143 (each its own causal end), 64 q heads / 4 groups, D=Di=128, "
                "bf16 q, e4m3 K/V/index keys, N(0,1), 8 planted blocks per seq, random "
                "permutation table")
    return w


def _prefill_chunk(name: str, cached: int, seed: int, kv_dtype: int = FP8, **kw) -> Workload:
    chunk = 4096
    w = make(name, seed=seed, seq_lens=[cached + chunk], rows_per_seq=chunk,
             q_pos=np.arange(cached, cached + chunk, dtype=np.int32), q_dtype=BF16,
             kv_dtype=kv_dtype, **kw)
    fmt = "e4m3" if kv_dtype == FP8 else "NVFP4 (quantised from N(0,1))"
    w.recipe = (f"chunked prefill: 1 seq, {cached} cached tokens + a 4096-query chunk at "
                f"positions {cached}..{cached + chunk - 1}, causal; 64 q heads / 4 groups, "
                f"D=Di=128, bf16 q, {fmt} K/V/index keys, N(0,1), random permutation table")
    return w


def prefill_64k(seed: int = 0x4D5341 + 6, **kw) -> Workload:
    return _prefill_chunk("prefill_64k", 65536, seed, **kw)


def prefill_64k_nvfp4(seed: int = 0x4D5341 + 6, **kw) -> Workload:
    """The prefill_64k chunk with NVFP4 K/V and index keys."""
    return _prefill_chunk("prefill_64k_nvfp4", 65536, seed, kv_dtype=NVFP4, **kw)


def prefill_16k(seed: int = 0x4D5341 + 6, **kw) -> Workload:
    """The prefill_64k chunk over 16,384 cached tokens: the same rows and
    blocks per row, a quarter of the K/V working set."""
    return _prefill_chunk("prefill_16k", 16384, seed, **kw)


def nvfp4_512k(seed: int = 0x4D5341 + 4, **kw) -> Workload:
    w = make("nvfp4_512k", seed=seed, seq_lens=[524288] * 4, q_dtype=BF16,
             kv_dtype=NVFP4, **kw)
    w.recipe = ("4 seqs x 524288 tokens, 64 q heads / 4 groups, D=Di=128, bf16 q, "
                "NVFP4 K/V/index keys quantised from N(0,1), random permutation table")
    return w
