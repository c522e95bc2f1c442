"""The C ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad problems on the host before any launch.  No call
here reaches a kernel."""
import ctypes
import os
import re

import pytest

import decode_msa_index_amd as msa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "msa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("msa_index_scores", "msa_block_topk", "msa_sparse_attend", "msa_decode"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = msa.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(msa.EXPORTS) == declared_functions()


def test_struct_layout_matches_header():
    # 15 int32 fields, 5 floats, the 2 forced-block counts, the share-group
    # size, no padding
    assert ctypes.sizeof(msa.MsaProblem) == 23 * 4
    assert msa.MsaProblem.init_blocks.offset == 20 * 4
    assert msa.MsaProblem.local_blocks.offset == 21 * 4
    assert msa.MsaProblem.share_seqs.offset == 22 * 4


def good(**kw):
    base = dict(num_seqs=2, max_blocks_per_seq=8, num_phys_blocks=16)
    base.update(kw)
    return msa.Problem(**base)


@pytest.mark.parametrize("op", [0, 1, 2, 3])
def test_valid_problem_passes(op):
    assert msa.check_problem(good(), op) == 0
    # forced blocks that fill the k exactly are fine
    assert msa.check_problem(good(top_k=8, init_blocks=3, local_blocks=5), op) == 0
    assert msa.check_problem(good(top_k=4, init_blocks=3, local_blocks=0), op) == 0
    # share groups: 0 and 1 mean none, up to 64 sequences per group
    for n in (0, 1, 2, 64):
        assert msa.check_problem(good(share_seqs=n), op) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(num_seqs=-1), 1), (dict(rows_per_seq=0), 1), (dict(num_q_heads=63), 1),
    (dict(max_blocks_per_seq=0), 1), (dict(num_phys_blocks=0), 1), (dict(top_k=0), 1),
    (dict(head_dim=64), 2), (dict(index_dim=256), 2), (dict(block_size=64), 2),
    (dict(top_k=33), 2), (dict(num_kv_groups=3, num_q_heads=48), 2),
    (dict(num_kv_groups=2, num_q_heads=64), 2),  # 32 heads per group
    (dict(index_k_dtype=1), 2), (dict(kv_dtype=1), 2), (dict(out_dtype=2), 2),
    (dict(index_q_dtype=0), 2), (dict(q_dtype=0), 2),
    (dict(sm_scale=0.0), 1), (dict(index_scale=-1.0), 1), (dict(k_scale=float("nan")), 1),
    (dict(num_seqs=20000), 2),
    (dict(init_blocks=-1), 1), (dict(local_blocks=-2), 1),
    (dict(top_k=16, init_blocks=16), 1),  # no place left for the recent block
    (dict(top_k=8, init_blocks=3, local_blocks=6), 1),
    (dict(share_seqs=-1), 1), (dict(share_seqs=65), 1),
    (dict(share_seqs=4, rows_per_seq=2), 2),  # share groups take one row per sequence
])
def test_bad_problems_rejected(kw, code):
    p = good(**kw)
    assert msa.check_problem(p, 3) == code
    assert msa.lib().msa_last_error() != b""


def test_null_and_misaligned_pointers_rejected_before_launch():
    p = good()
    with pytest.raises(msa.MsaError) as e:
        msa.index_scores(p, None, None, None, None, None, None, None, stream=0)
    assert e.value.status == 1 and "index_q" in e.value.detail
    with pytest.raises(msa.MsaError) as e:
        msa.index_scores(p, 0x1001, 0x2000, None, 0x3000, 0x4000, None, 0x5000, stream=0)
    assert e.value.status == 1 and "aligned" in e.value.detail
    with pytest.raises(msa.MsaError) as e:  # rows_per_seq > 1 needs positions
        msa.block_topk(good(rows_per_seq=2), 0x1000, 0x2000, None, 0x3000, stream=0)
    assert e.value.status == 1
    with pytest.raises(msa.MsaError) as e:  # nvfp4 needs scales
        msa.sparse_attend(good(kv_dtype=3), 0x1000, 0x2000, None, 0x3000, 0x4000, None,
                          0x5000, 0x6000, None, None, stream=0)
    assert e.value.status == 1 and "kv_scales" in e.value.detail
    with pytest.raises(msa.MsaError) as e:  # outputs are written 16 bytes at a time
        msa.sparse_attend(good(), 0x1000, 0x2000, None, 0x3000, 0x4000, None,
                          0x5000, 0x6008, None, None, stream=0)
    assert e.value.status == 1 and "out" in e.value.detail and "aligned" in e.value.detail


def test_workspace_sizes():
    p = good(num_seqs=8, max_blocks_per_seq=2049)
    assert msa.workspace_bytes(p, msa.OP_INDEX) == 0
    assert msa.workspace_bytes(p, msa.OP_TOPK) == 0
    a = msa.workspace_bytes(p, msa.OP_ATTEND)
    d = msa.workspace_bytes(p, msa.OP_DECODE)
    scores = 8 * 4 * 2049 * 4
    zone_end = 256 + 512 * 16 * 130 * 4  # the status header and the split-K zone
    assert d % 256 == 0 and a % 256 == 0
    # decode: the pooled scores (rounded up to 256) after the status header
    # and the whole split zone, which every call leaves zero
    assert a < zone_end and d == zone_end + -(-scores // 256) * 256
    # a 256-byte status header, then the split partials: 16 heads x (128
    # outputs + max + denominator) per split
    units = 8 * 4
    S = (a - 256) // (units * 16 * 130 * 4)
    assert S >= 2 and a == 256 + -(-(units * S * 16 * 130 * 4) // 256) * 256
    big = good(num_seqs=512, max_blocks_per_seq=16)
    assert msa.workspace_bytes(big, msa.OP_ATTEND) == 0  # enough (row, group)s: no split
    assert msa.workspace_bytes(big, msa.OP_DECODE) == zone_end + 512 * 4 * 16 * 4


def test_workspace_sizes_of_the_key_block_path():
    """A chunk of 640+ rows per sequence over an FP8 or NVFP4 cache takes
    the key-block attention, whose workspace holds, after the status header
    and the split-K zone, per (row, group, slot) a 4 KB f16 partial, a
    128-byte (max, sum) record and two list words, plus per-slice and
    per-block arrays and the chunk table; 639 rows take the per-row
    kernel, which needs none at 512+ (row, group) units."""
    def sizes(R, kv=2):
        p = good(num_seqs=1, rows_per_seq=R, max_blocks_per_seq=544, num_phys_blocks=544,
                 kv_dtype=kv)
        return msa.workspace_bytes(p, msa.OP_ATTEND), msa.workspace_bytes(p, msa.OP_DECODE)
    assert sizes(639)[0] == 0
    for kv in (2, 3):
        a, d = sizes(4096, kv)
        slots = 4096 * 4 * 16
        per_slot = 4096 + 128 + 8
        zone = 512 * 16 * 130 * 4  # the split-K zone, which the path leaves alone
        assert slots * per_slot < a - 256 - zone < slots * per_slot * 1.002
        # decode adds the pooled scores
        assert d - a == -(-(4096 * 4 * 544 * 4) // 256) * 256
    a640, _ = sizes(640)
    assert a640 > 640 * 4 * 16 * (4096 + 128 + 8)


def test_status_strings():
    L = msa.lib()
    assert L.msa_status_string(0) == b"ok"
    assert L.msa_status_string(3) == b"workspace too small"
    assert L.msa_status_string(5) == b"a device-side wait gave up"


def test_cache_write_rejects_bad_arguments_before_launch():
    p = good(num_seqs=2, max_blocks_per_seq=4)
    ok = dict(token_seq=0x1000, token_pos=0x2000, k_new=0x3000, v_new=0x4000, ik_new=0x5000,
              block_table=0x6000, kv_data=0x7000, kv_scales=None, ik_data=0x8000,
              ik_scales=None)
    L = msa.lib()

    def call(n, **kw):
        a = dict(ok, **kw)
        return L.msa_cache_write(ctypes.byref(p.c()), n, a["token_seq"], a["token_pos"],
                                 a["k_new"], a["v_new"], a["ik_new"], a["block_table"],
                                 a["kv_data"], a["kv_scales"], a["ik_data"], a["ik_scales"],
                                 None)
    assert call(0) == 0  # nothing to write: no launch, no pointer needed
    assert call(-1) == 1
    assert call(70000) == 2
    assert call(3, k_new=None) == 1
    assert call(3, kv_data=0x7008) == 1  # misaligned
    p4 = good(num_seqs=2, max_blocks_per_seq=4, kv_dtype=msa.NVFP4)
    assert L.msa_cache_write(ctypes.byref(p4.c()), 3, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000,
                             0x6000, 0x7000, None, 0x8000, None, None) == 1  # scales missing
    assert msa.check_problem(p, msa.OP_CACHE_WRITE) == 0
