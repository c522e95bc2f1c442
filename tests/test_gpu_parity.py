"""GPU parity of every call of the C ABI against the CPU oracle.

Inputs are seeded synthetic workloads (synth); expected values come from the
oracle only.  Small cases span several blocks, ragged tails and the
degenerate cases; the full-size cases are the benchmark's workloads in the
benchmark's launch configuration, with the oracle computed on every output.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_msa_index_amd as msa


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.lib()


def _oracle_all(w, threads=0):
    p = parity.oracle_problem(w, threads)
    return oracle.decode(p, w.index_q, w.ik_data, w.ik_scales, w.q, w.kv_data, w.kv_scales,
                         w.block_table, w.seq_lens, w.q_pos)


def _run_and_check(w, fused, name, ref=None):
    """ref: the oracle's (scores, selection, out, lse) of w, when the caller
    already has them."""
    if ref is None:
        say(f"[parity] {name}: oracle on {w.rows} rows")
        ref = _oracle_all(w)
    s_ref, k_ref, o_ref, l_ref = ref
    dw = parity.DeviceWorkload(w)
    say(f"[parity] {name}: GPU {'msa_decode' if fused else 'three-call chain'}")
    if fused:
        dw.decode()
    else:
        dw.chain()
    torch.cuda.synchronize()
    s = dw.scores.cpu().numpy()
    k = dw.topk.cpu().numpy()
    o = dw.out.float().cpu().numpy()
    serr = parity.check_scores(w, s, s_ref)
    same = parity.check_selection(w, s_ref, k_ref, k)
    aerr = parity.check_decode_attention(w, o, o_ref, same, k)
    parity.record(name, same, serr, aerr)
    say(f"[parity] {name}: score err {serr:.3f} of bound, {int(same.sum())}/{same.size} "
        f"selections identical, attention max-abs {aerr:.2e} (every unit)")
    return dw, same


# ---------------------------------------------------------------------------
# small, several tiles, ragged tails, edge cases
# ---------------------------------------------------------------------------

EDGE_LENS = [1, 127, 128, 129, 2047, 2048, 2049, 16 * 128 + 1, 5000, 130 * 128 - 3]


@pytest.mark.parametrize("kv", [synth.FP8, synth.NVFP4])
@pytest.mark.parametrize("fused", [False, True])
def test_small_ragged(kv, fused):
    w = synth.make("edge", seed=101 + kv, seq_lens=EDGE_LENS, q_dtype=synth.BF16,
                   kv_dtype=kv, plant_per_seq=0)
    _run_and_check(w, fused, f"edge-{synth.DTYPE_NAMES[kv]}")


def _scale_bf16(bits: np.ndarray, k: int) -> np.ndarray:
    """bf16 bit patterns times 2**k, exactly (zeros stay zero)."""
    b = bits.astype(np.uint32)
    e = (b >> 7) & 0xFF
    ne = (e.astype(np.int64) + k).astype(np.uint32)
    assert np.all((ne[e > 0] >= 1) & (ne[e > 0] <= 254)), "scaled out of bf16's range"
    return np.where(e > 0, (b & np.uint32(0x807F)) | (ne << 7), b).astype(np.uint16)


@pytest.mark.parametrize("kv", [synth.FP8, synth.NVFP4])
def test_index_queries_far_outside_f16_range(kv):
    # NVFP4 keys are scored on f16 MFMA with each index query shifted by a
    # power of two into f16's range; these queries would overflow (2^60),
    # flush to zero (2^-60) or lose bits (a 2^30 spread inside one query)
    # without the shift.  One group's query is zero: all its blocks tie at 0.
    w = synth.make("iq-range", seed=171 + kv, seq_lens=[5000, 2049, 3000, 700],
                   q_dtype=synth.BF16, kv_dtype=kv, plant_per_seq=2)
    iq = w.index_q.copy()
    iq[0] = _scale_bf16(iq[0], 60)
    iq[1] = _scale_bf16(iq[1], -60)
    iq[2, 1] = 0
    iq[3, :, :64] = _scale_bf16(iq[3, :, :64], 20)
    iq[3, :, 64:] = _scale_bf16(iq[3, :, 64:], -10)
    w = dataclasses.replace(w, index_q=iq)
    for fused in (False, True):
        _, same = _run_and_check(w, fused, f"iq-range-{synth.DTYPE_NAMES[kv]}")
        assert same[2, 1], "a zero query selects the lowest blocks on both sides"


def _decode_outputs(w):
    dw = parity.DeviceWorkload(w)
    dw.decode()
    torch.cuda.synchronize()
    return dw.scores.cpu(), dw.topk.cpu(), dw.out.cpu()


@pytest.mark.parametrize("kv,n,G,H,share_blocks,diverge", [
    (synth.FP8, 16, 4, 64, 60, False),    # one full group of 16 and a group of 4
    (synth.FP8, 5, 4, 64, 40, True),      # a member leaves the prefix half way
    (synth.NVFP4, 5, 4, 64, 40, False),
    (synth.FP8, 64, 1, 16, 20, False),    # 64 sequences on one wave's columns
    (synth.FP8, 8, 8, 64, 30, False),
    (synth.FP8, 16, 4, 64, 0, False),     # the hint over unshared random tables
    (synth.NVFP4, 16, 4, 64, 60, "qpos"),  # rows ending inside the shared prefix
])
def test_shared_prefix_scan(kv, n, G, H, share_blocks, diverge):
    # requests with common prefixes: the index scan reads each distinct
    # physical block once per share group slice; the scores, selection and
    # output must be the oracle's, and bit for bit those of the unshared scan
    nseq = n + 4 if n < 64 else 64
    rng = np.random.default_rng(200 + n + G)
    lens = [int(share_blocks * 128 + rng.integers(1, 2000)) for _ in range(nseq)]
    if n < 64:
        lens[-1] = 300  # a short member: sees only the first blocks of the prefix
    w = synth.make(f"share-{n}", seed=210 + n + G + kv, seq_lens=lens, num_q_heads=H,
                   num_groups=G, q_dtype=synth.BF16, kv_dtype=kv, plant_per_seq=2,
                   share_seqs=n, share_blocks=share_blocks)
    if share_blocks == 0:
        w = dataclasses.replace(w, share_seqs=n)
    if diverge == "qpos":  # query rows at earlier positions, some deep inside the prefix
        qp = np.array([L - 1 - (rng.integers(0, L) if b % 3 == 0 else 0)
                       for b, L in enumerate(lens)], np.int32)
        w = dataclasses.replace(w, q_pos=qp)
    elif diverge:  # member 1 takes member 2's private blocks for part of the prefix
        bt = w.block_table.copy()
        nb2 = (lens[2] + 127) // 128
        k = min(10, nb2 - share_blocks)
        bt[1, 20: 20 + k] = bt[2, share_blocks: share_blocks + k]
        w = dataclasses.replace(w, block_table=bt)
    shared = int(sum((w.block_table[b, :share_blocks] == w.block_table[(b // n) * n, :share_blocks]).sum()
                     for b in range(nseq)))
    say(f"[parity] share-{n}: {nseq} sequences, {shared} (sequence, block) entries shared")
    _run_and_check(w, True, f"share-{n}-{synth.DTYPE_NAMES[kv]}")
    _run_and_check(w, False, f"share-{n}-{synth.DTYPE_NAMES[kv]}-chain")
    s1, k1, o1 = _decode_outputs(w)
    s0, k0, o0 = _decode_outputs(dataclasses.replace(w, share_seqs=0))
    assert torch.equal(s1.view(torch.int32), s0.view(torch.int32)), "shared scan scores differ"
    assert torch.equal(k1, k0) and torch.equal(o1.view(torch.int16), o0.view(torch.int16))


def test_context_shards_merge_to_the_full_selection():
    # Context parallelism of the indexer (the pages' DCP): shard k of 4 holds
    # a contiguous quarter of every sequence's blocks and scores it with its
    # own block table.  Each shard's pooled scores must be those of the full
    # scan, bit for bit, and the shards' local top-(k-1) candidates
    # (score desc, block asc), merged, must give the full selection.
    w = synth.make("dcp", seed=230, seq_lens=[20000, 9000, 16385], q_dtype=synth.BF16,
                   kv_dtype=synth.FP8, plant_per_seq=3)
    dw = parity.DeviceWorkload(w)
    dw.index_scores()
    dw.block_topk()
    torch.cuda.synchronize()
    full = dw.scores.cpu().numpy()
    sel = dw.topk.cpu().numpy()
    nb = (w.seq_lens.astype(np.int64) + 127) // 128
    K, S = w.top_k, 4
    cands = [[[] for _ in range(w.num_groups)] for _ in range(w.num_seqs)]
    for k in range(S):
        lo = [int(k * n // S) for n in nb]
        hi = [int((k + 1) * n // S) for n in nb]
        mbk = max(1, max(h - l for l, h in zip(lo, hi)))
        bt = np.zeros((w.num_seqs, mbk), np.int32)
        lens = np.zeros(w.num_seqs, np.int32)
        for b in range(w.num_seqs):
            bt[b, : hi[b] - lo[b]] = w.block_table[b, lo[b]: hi[b]]
            lens[b] = max(0, min(int(w.seq_lens[b]) - 128 * lo[b], 128 * (hi[b] - lo[b])))
        p = dataclasses.replace(dw.p, max_blocks_per_seq=mbk)
        sk = torch.empty(w.num_seqs, w.num_groups, mbk, dtype=torch.float32, device="cuda")
        msa.index_scores(p, dw.index_q, dw.ik_data, dw.ik_scales, parity.dev(bt),
                         parity.dev(lens), None, sk)
        torch.cuda.synchronize()
        sk = sk.cpu().numpy()
        for b in range(w.num_seqs):
            n = hi[b] - lo[b]
            got, want = sk[b, :, :n], full[b, :, lo[b]: hi[b]]
            assert np.array_equal(got.view(np.int32), want.view(np.int32)), (k, b)
            for g in range(w.num_groups):  # local candidates, the recent block excluded
                js = [j for j in range(lo[b], hi[b]) if j != nb[b] - 1]
                js.sort(key=lambda j: (-float(full[b, g, j]), j))
                cands[b][g] += [(float(full[b, g, j]), j) for j in js[: K - 1]]
    for b in range(w.num_seqs):
        for g in range(w.num_groups):
            merged = sorted(cands[b][g], key=lambda c: (-c[0], c[1]))[: K - 1]
            want = sorted([j for _, j in merged] + [int(nb[b] - 1)])
            assert [int(x) for x in sel[b, g] if x >= 0] == want, (b, g)


def test_tiny_fp32_workload():
    w = synth.tiny()
    dw, same = _run_and_check(w, fused=False, name="tiny-f32")
    assert same.all()


def test_tiny_fp32_output():
    w = synth.tiny()
    s_ref, k_ref, o_ref, l_ref = _oracle_all(w)
    dw = parity.DeviceWorkload(w, out_dtype=msa.F32)
    say("[parity] tiny f32 out")
    dw.chain()
    torch.cuda.synchronize()
    o = dw.out.cpu().numpy()
    assert np.array_equal(dw.topk.cpu().numpy(), k_ref)
    assert np.max(np.abs(o - o_ref)) < 1e-4
    np.testing.assert_allclose(dw.lse.cpu().numpy(), l_ref, rtol=0, atol=1e-4)


@pytest.mark.parametrize("G,H", [(1, 16), (2, 8), (8, 8), (4, 12)])
def test_group_shapes(G, H):
    w = synth.make("groups", seed=7 + G + H, seq_lens=[3000, 700, 129], num_q_heads=H,
                   num_groups=G, q_dtype=synth.BF16, kv_dtype=synth.FP8, top_k=8)
    _run_and_check(w, fused=True, name=f"G{G}H{H}")


@pytest.mark.parametrize("K", [1, 4, 8, 32])
def test_topk_sizes(K):
    w = synth.make("topk", seed=50 + K, seq_lens=[6000, 128 * 40, 300], q_dtype=synth.BF16,
                   kv_dtype=synth.FP8, top_k=K)
    _run_and_check(w, fused=True, name=f"K{K}")


def test_query_positions_multi_row():
    lens = [4000, 2600]
    qp = np.array([3999, 3000, 1, 128, 2599, 2047], np.int32)
    w = synth.make("rows", seed=77, seq_lens=lens, rows_per_seq=3, q_pos=qp,
                   q_dtype=synth.BF16, kv_dtype=synth.FP8, top_k=4)
    _run_and_check(w, fused=True, name="multi-row")


@pytest.mark.parametrize("kv,R,G,H", [(synth.FP8, 4, 4, 64), (synth.NVFP4, 4, 4, 64),
                                       (synth.FP8, 6, 4, 64), (synth.FP8, 5, 2, 16),
                                       (synth.FP8, 3, 8, 64)])
def test_speculative_rows_share_one_scan(kv, R, G, H):
    """Several query rows per sequence (speculative decode: the last R
    positions, each row with its own causal end and recent block): the scan
    scores up to 16 / G rows per pass over the keys (R = 6 with G = 4: two
    row groups, of 4 and 2 rows), and every row matches the oracle."""
    lens = [9000, 4100, 129, 20000]
    qp = np.concatenate([np.arange(L - R, L) for L in lens]).astype(np.int32)
    qp[R] = 5  # one row far behind the others of its sequence
    w = synth.make(f"spec-r{R}", seed=120 + R + kv, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                   num_q_heads=H, num_groups=G, q_dtype=synth.BF16, kv_dtype=kv,
                   plant_per_seq=2)
    _run_and_check(w, fused=True, name=f"spec-r{R}-g{G}-{synth.DTYPE_NAMES[kv]}")


# (MB, B): the selection kernel's three forms -- one wave per unit (short
# rows, or 512 and more units), a four-wave workgroup per unit (few units on
# long rows), and the radix workgroup for rows too long for LDS
TOPK_FORMS = [(300, 9), (700, 9), (700, 130), (17000, 9)]


@pytest.mark.parametrize("MB,B", TOPK_FORMS)
def test_block_topk_bit_exact_with_ties(MB, B):
    """Selection kernel alone, on oracle-independent scores with many exact
    ties: identical to the oracle's selection, in each of the kernel's
    forms."""
    rng = np.random.default_rng(5)
    G = 4
    lens = rng.integers(1, min(MB, 3000) * 128 + 1, B).astype(np.int32)
    lens[0], lens[1], lens[2] = min(MB, 3000) * 128, 1, 17 * 128
    scores = rng.integers(-6, 7, (B, G, MB)).astype(np.float32) * 0.25
    scores[3] = -0.0  # signed zeros tie with +0
    scores[3, :, ::3] = 0.0
    # every 8th block high: the high blocks sit in few lanes of the wave-level
    # selection, more than 64 candidates clear its first threshold, and it
    # takes its radix path
    scores[4] = rng.standard_normal((G, MB)).astype(np.float32) * 1e-3
    scores[4, :, ::8] += 1.0 + rng.random((G, (MB + 7) // 8)).astype(np.float32)
    lens[4] = min(MB, 3000) * 128
    for K in (1, 5, 16, 32):
        op = oracle.Problem(num_seqs=B, num_q_heads=G, num_groups=G, block_size=128, top_k=K,
                            max_blocks=MB, num_phys_blocks=1)
        ref = oracle.block_topk(op, scores, lens)
        p = msa.Problem(num_seqs=B, num_q_heads=G, num_kv_groups=G, top_k=K,
                        max_blocks_per_seq=MB, num_phys_blocks=1)
        out = torch.empty(B, G, K, dtype=torch.int32, device="cuda")
        say(f"[parity] block_topk K={K}")
        msa.block_topk(p, parity.dev(scores), parity.dev(lens), None, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("MB,B", [(mb, 2 * b) for mb, b in TOPK_FORMS])
def test_block_topk_forced_blocks_bit_exact(MB, B):
    """Leading (init) and trailing (local) blocks always kept: the selection
    kernel alone matches the oracle exactly, for every top-k the attention
    accepts, forced sets that leave few or no free places, and the score
    pattern that sends the wave-level selection down its radix path, in each
    of the kernel's forms."""
    rng = np.random.default_rng(6)
    G = 2
    n = min(MB, 3000)
    lens = rng.integers(1, n * 128 + 1, B).astype(np.int32)
    lens[0], lens[1], lens[2], lens[3] = n * 128, 1, 9 * 128, 33 * 128 + 1
    scores = rng.integers(-6, 7, (B, G, MB)).astype(np.float32) * 0.25
    scores[4] = rng.standard_normal((G, MB)).astype(np.float32) * 1e-3
    scores[4, :, ::8] += 1.0 + rng.random((G, (MB + 7) // 8)).astype(np.float32)
    lens[4] = n * 128
    for K, init, local in [(4, 1, 1), (8, 2, 4), (16, 1, 3), (16, 4, 0), (32, 8, 8),
                           (8, 7, 1), (16, 0, 16), (32, 1, 2)]:
        op = oracle.Problem(num_seqs=B, num_q_heads=G, num_groups=G, block_size=128, top_k=K,
                            max_blocks=MB, num_phys_blocks=1, init_blocks=init,
                            local_blocks=local)
        ref = oracle.block_topk(op, scores, lens)
        p = msa.Problem(num_seqs=B, num_q_heads=G, num_kv_groups=G, top_k=K,
                        max_blocks_per_seq=MB, num_phys_blocks=1, init_blocks=init,
                        local_blocks=local)
        out = torch.full((B, G, K), 7, dtype=torch.int32, device="cuda")
        say(f"[parity] block_topk MB={MB} K={K} init={init} local={local}")
        msa.block_topk(p, parity.dev(scores), parity.dev(lens), None, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), (K, init, local)


@pytest.mark.parametrize("K,init,local", [(16, 2, 4), (8, 1, 2), (32, 4, 8), (4, 3, 1)])
@pytest.mark.parametrize("fused", [False, True])
def test_decode_with_forced_blocks(K, init, local, fused):
    """Decode with leading and trailing blocks always kept: selection (with
    the near-tie rule for the free places) and attention match the oracle,
    through the fused decode and through the three-call chain."""
    base = synth.make("forced", seed=140 + K + init, seq_lens=[20000, 9000, 3 * 128 + 5, 1100],
                      q_dtype=synth.BF16, kv_dtype=synth.FP8, plant_per_seq=3, top_k=K)
    w = dataclasses.replace(base, init_blocks=init, local_blocks=local)
    dw, same = _run_and_check(w, fused, f"forced-k{K}-i{init}-l{local}")
    topk = dw.topk.cpu().numpy()
    for r in range(w.rows):
        rb = (int(w.seq_lens[r]) - 1) // 128
        for g in range(w.num_groups):
            sel = set(int(x) for x in topk[r, g] if x >= 0)
            if rb + 1 > K:
                assert set(range(init)) <= sel
                assert set(range(rb + 1 - max(local, 1), rb + 1)) <= sel


def test_sparse_attend_on_oracle_selection():
    """Attention kernel alone, fed the oracle's selection."""
    w = synth.make("attend", seed=31, seq_lens=[9000, 2100, 128], q_dtype=synth.BF16,
                   kv_dtype=synth.FP8)
    s_ref, k_ref, o_ref, l_ref = _oracle_all(w)
    dw = parity.DeviceWorkload(w)
    say("[parity] sparse_attend on oracle selection")
    dw.sparse_attend(topk=parity.dev(k_ref))
    torch.cuda.synchronize()
    parity.check_attention(w, dw.out.float().cpu().numpy(), o_ref)
    np.testing.assert_allclose(dw.lse.cpu().numpy(), l_ref, rtol=0, atol=2e-3)


def test_decode_equals_chain_and_is_deterministic():
    """The fused decode makes the same selection as the three-kernel chain,
    stores the same scores and attends the selected blocks in the same
    (ascending) order with the same launch shape, so its outputs and lse are
    bit-identical to the chain's, on a shape that splits each (row, group)
    over several workgroups and on one that does not.  Repeated decodes are
    bit-identical."""
    for lens in ([20000, 7000, 300], [9000] * 80):
        w = synth.make("det", seed=44, seq_lens=lens, q_dtype=synth.BF16,
                       kv_dtype=synth.FP8, plant_per_seq=4)
        dw = parity.DeviceWorkload(w)
        say(f"[parity] chain vs decode vs decode, {len(lens)} sequences")
        dw.chain()
        torch.cuda.synchronize()
        chain = (dw.scores.clone(), dw.topk.clone(), dw.out.view(torch.uint8).clone(),
                 dw.lse.clone())
        first = None
        for with_scores in (True, True, False):
            dw.decode(with_scores=with_scores)
            torch.cuda.synchronize()
            if with_scores:
                assert torch.equal(dw.scores, chain[0])
            assert torch.equal(dw.topk, chain[1])
            assert torch.equal(dw.out.view(torch.uint8), chain[2]), "decode out != chain out"
            assert torch.equal(dw.lse, chain[3]), "decode lse != chain lse"
            now = (dw.topk.clone(), dw.out.view(torch.uint8).clone(), dw.lse.clone())
            if first is None:
                first = now
            else:
                assert all(torch.equal(x, y) for x, y in zip(first, now)), "decode not deterministic"
            assert int(torch.count_nonzero(dw.ws_decode[:SPLIT_ZONE_BYTES])) == 0, "workspace not left zero-filled"


def test_decode_in_graph_replays_match_eager():
    """msa_decode captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, reproduces the eager results bit for
    bit and leaves the workspace zero-filled."""
    w = synth.make("graph", seed=71, seq_lens=[20000, 9000, 300, 65536], q_dtype=synth.BF16,
                   kv_dtype=synth.FP8, plant_per_seq=2)
    dw = parity.DeviceWorkload(w)
    dw.decode(with_scores=True)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (dw.scores, dw.topk, dw.out, dw.lse)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dw.decode(with_scores=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dw.decode(with_scores=True)
    for rep in range(4):
        say(f"[parity] graph replay {rep}")
        dw.scores.zero_()
        dw.topk.fill_(-7)
        dw.out.zero_()
        dw.lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(ref, (dw.scores, dw.topk, dw.out, dw.lse)):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)
        assert int(torch.count_nonzero(dw.ws_decode[:SPLIT_ZONE_BYTES])) == 0


def test_repeated_decode_never_stalls():
    """Split-K units merge by polling: many decodes in a row (every wave of
    the merging workgroup polls the shared max / denominator words, which
    may only be cleared once all of them are done) all finish promptly with
    finite, identical outputs."""
    import time
    w = synth.make("repeat", seed=81, seq_lens=EDGE_LENS, q_dtype=synth.BF16,
                   kv_dtype=synth.FP8, plant_per_seq=2)
    dw = parity.DeviceWorkload(w)
    dw.decode(with_scores=False)
    torch.cuda.synchronize()
    ref = dw.out.view(torch.uint8).clone()
    say("[parity] 40 decodes in a row")
    t0 = time.perf_counter()
    for _ in range(40):
        dw.decode(with_scores=False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert elapsed < 0.5, f"40 decodes took {elapsed:.3f} s: a merge waited for its spin limit"
    assert torch.isfinite(dw.out.float()).all()
    assert torch.equal(dw.out.view(torch.uint8), ref)
    assert int(torch.count_nonzero(dw.ws_decode[:SPLIT_ZONE_BYTES])) == 0


def test_nan_in_cache_reaches_the_output_without_stalling_the_merge():
    """A NaN in V (e4m3 0x7F) at token 0 of every block of one (sequence,
    group), dim 5: every split's partial for that dim is NaN, the merge
    still completes at once (partials carry NaNs in a form that is never
    the all-zero 'not yet written' word), the NaN reaches exactly that
    dim of that group's heads, and every other output is unchanged."""
    import time
    w = synth.make("nanv", seed=91, seq_lens=[20000, 9000], q_dtype=synth.BF16,
                   kv_dtype=synth.FP8, plant_per_seq=2)
    dw = parity.DeviceWorkload(w)
    dw.decode(with_scores=False)
    torch.cuda.synchronize()
    ref = dw.out.float().clone()
    b, g, d = 0, 1, 5
    nb = -(-int(w.seq_lens[b]) // 128)
    pbs = torch.from_numpy(w.block_table[b, :nb].astype(np.int64)).cuda()
    dw.kv_data[pbs, 1, g, d, 0] = 0x7F
    torch.cuda.synchronize()
    say("[parity] decode with a NaN in V")
    t0 = time.perf_counter()
    dw.decode(with_scores=False)
    torch.cuda.synchronize()
    assert time.perf_counter() - t0 < 0.2, "the split-K merge waited for its spin limit"
    out = dw.out.float()
    hpg = w.num_q_heads // w.num_groups
    heads = slice(g * hpg, (g + 1) * hpg)
    assert torch.isnan(out[b, heads, d]).all()
    mask = torch.ones_like(out, dtype=torch.bool)
    mask[b, heads, d] = False
    assert torch.equal(out[mask], ref[mask])
    assert int(torch.count_nonzero(dw.ws_decode[:SPLIT_ZONE_BYTES])) == 0


def _cache_write_inputs(kv, ik, q_dtype, iq_dtype, seed, spikes=True, G=4, H=64):
    lens = [900, 300, 129, 5000]
    w = synth.make("cw", seed=seed, seq_lens=lens, q_dtype=q_dtype, index_q_dtype=iq_dtype,
                   kv_dtype=kv, index_k_dtype=ik, k_scale=0.75, v_scale=1.25,
                   ik_scale=0.5 if ik != synth.NVFP4 else None, plant_per_seq=1,
                   num_groups=G, num_q_heads=H)
    # block boundaries, both tokens of a V nibble pair, a sequence's last
    # key, and tokens out of range (skipped)
    seq = np.array([0, 0, 0, 1, 1, 2, 2, 3, 3, 3, -1, 4, 0], np.int32)
    pos = np.array([0, 1, 899, 128, 129, 127, 128, 4998, 4999, 2500, 5, 5,
                    w.max_blocks * 128], np.int32)
    rng = np.random.default_rng(seed)
    n, G, D = len(seq), w.num_groups, w.head_dim

    # with spikes: a wide spread and saturating values (the write's edge
    # cases); without: the cached values' own N(0, 1) scale, since the
    # attention bound of the decode that follows is absolute (bf16 rounding
    # alone exceeds 1e-2 on outputs of magnitude 4 and more)
    sigma = 2.0 if spikes else 1.0

    def vals(*shape):
        x = rng.normal(0, sigma, shape) * np.where(rng.random(shape) < 0.1, 1e-3, 1.0)
        if spikes:
            x[rng.random(shape) < 0.01] = 3000.0  # saturating values
        return x.astype(np.float32)

    enc = lambda x, dt: x if dt == synth.F32 else synth.encode_bf16(x)
    new = dict(k=enc(vals(n, G, D), q_dtype), v=enc(vals(n, G, D), q_dtype),
               ik=enc(vals(n, w.index_dim), iq_dtype))
    return w, seq, pos, new


@pytest.mark.parametrize("kv,ik,q,iq", [(synth.FP8, synth.FP8, synth.BF16, synth.BF16),
                                        (synth.NVFP4, synth.NVFP4, synth.BF16, synth.BF16),
                                        (synth.F32, synth.F32, synth.F32, synth.F32),
                                        (synth.FP8, synth.NVFP4, synth.BF16, synth.BF16)])
def test_cache_write_is_bit_exact_with_the_oracle(kv, ik, q, iq):
    w, seq, pos, new = _cache_write_inputs(kv, ik, q, iq, seed=31 + kv + 4 * ik)
    ref = {k: (None if getattr(w, k) is None else getattr(w, k).copy())
           for k in ("kv_data", "kv_scales", "ik_data", "ik_scales")}
    oracle.cache_write(parity.oracle_problem(w), seq, pos, new["k"], new["v"], new["ik"],
                       w.block_table, ref["kv_data"], ref["kv_scales"], ref["ik_data"],
                       ref["ik_scales"])
    dw = parity.DeviceWorkload(w)
    say(f"[parity] cache write kv={kv} ik={ik}")
    msa.cache_write(dw.p, parity.dev(seq), parity.dev(pos), parity.dev(new["k"]),
                    parity.dev(new["v"]), parity.dev(new["ik"]), dw.block_table, dw.kv_data,
                    dw.kv_scales, dw.ik_data, dw.ik_scales)
    torch.cuda.synchronize()
    for name in ("kv_data", "kv_scales", "ik_data", "ik_scales"):
        if ref[name] is None:
            continue
        got = getattr(dw, name).cpu().numpy().view(np.uint8)
        want = ref[name].view(np.uint8)
        assert np.array_equal(got, want), f"{name}: {int((got != want).sum())} bytes differ"
    assert not np.array_equal(ref["kv_data"], w.kv_data)  # the write changed something


@pytest.mark.parametrize("kv,G,H", [(synth.FP8, 4, 64), (synth.NVFP4, 4, 64), (synth.F32, 4, 64),
                                    (synth.FP8, 8, 64), (synth.NVFP4, 1, 16), (synth.F32, 2, 16)])
def test_cache_write_runs_are_bit_exact(kv, G, H):
    # V is stored transposed; aligned runs of 16 consecutive positions of one
    # sequence are written a dim row at a time, everything else token by
    # token.  The list mixes both: aligned runs over two blocks, runs that
    # start 16 before and at a block edge, misaligned runs, a reversed run, a
    # run broken by a skipped entry, and a short tail.
    q = synth.F32 if kv == synth.F32 else synth.BF16
    w, _, _, _ = _cache_write_inputs(kv, kv, q, q, seed=60 + kv + G, G=G, H=H)
    # (lists of 512 entries or more take the run path: this one has 613)
    parts = [(3, np.arange(1024, 1536)), (0, np.arange(8, 40)), (3, np.arange(112, 144)),
             (1, np.arange(15, -1, -1)), (3, np.arange(2000, 2016)), (2, np.arange(0, 5))]
    seq = np.concatenate([np.full(len(p_), s_, np.int32) for s_, p_ in parts])
    pos = np.concatenate([p_ for _, p_ in parts]).astype(np.int32)
    assert len(seq) >= 512
    seq[sum(len(p_) for _, p_ in parts[:4]) + 7] = -1  # breaks the run at 2000 (entry skipped)
    rng = np.random.default_rng(61 + kv)
    n, G, D = len(seq), w.num_groups, w.head_dim
    enc = lambda x: x.astype(np.float32) if q == synth.F32 else synth.encode_bf16(x)
    new = dict(k=enc(rng.normal(0, 2.0, (n, G, D))), v=enc(rng.normal(0, 2.0, (n, G, D))),
               ik=enc(rng.normal(0, 2.0, (n, w.index_dim))))
    ref = {k: (None if getattr(w, k) is None else getattr(w, k).copy())
           for k in ("kv_data", "kv_scales", "ik_data", "ik_scales")}
    oracle.cache_write(parity.oracle_problem(w), seq, pos, new["k"], new["v"], new["ik"],
                       w.block_table, ref["kv_data"], ref["kv_scales"], ref["ik_data"],
                       ref["ik_scales"])
    dw = parity.DeviceWorkload(w)
    say(f"[parity] cache write runs kv={kv}: {n} tokens")
    msa.cache_write(dw.p, parity.dev(seq), parity.dev(pos), parity.dev(new["k"]),
                    parity.dev(new["v"]), parity.dev(new["ik"]), dw.block_table, dw.kv_data,
                    dw.kv_scales, dw.ik_data, dw.ik_scales)
    torch.cuda.synchronize()
    for name in ("kv_data", "kv_scales", "ik_data", "ik_scales"):
        if ref[name] is None:
            continue
        got = getattr(dw, name).cpu().numpy().view(np.uint8)
        want = ref[name].view(np.uint8)
        assert np.array_equal(got, want), f"{name}: {int((got != want).sum())} bytes differ"


def test_cache_write_then_decode_sees_the_new_tokens():
    """A decode step end to end: write every sequence's newest token (and a
    few older ones) into FP8 caches, then msa_decode; the oracle decodes
    the caches its own write produced, and the two agree.  (Values of
    ordinary magnitude: the attention bound is absolute.)"""
    w, seq, pos, new = _cache_write_inputs(synth.FP8, synth.FP8, synth.BF16, synth.BF16,
                                           seed=77, spikes=False)
    keep = (seq >= 0) & (seq < w.num_seqs) & (pos < w.max_blocks * 128)
    seq, pos = seq[keep], pos[keep]
    new = {k: np.ascontiguousarray(v[keep]) for k, v in new.items()}
    ref = {k: getattr(w, k).copy() for k in ("kv_data", "ik_data")}
    oracle.cache_write(parity.oracle_problem(w), seq, pos, new["k"], new["v"], new["ik"],
                       w.block_table, ref["kv_data"], None, ref["ik_data"], None)
    dw = parity.DeviceWorkload(w)
    msa.cache_write(dw.p, parity.dev(seq), parity.dev(pos), parity.dev(new["k"]),
                    parity.dev(new["v"]), parity.dev(new["ik"]), dw.block_table, dw.kv_data,
                    None, dw.ik_data, None)
    w2 = dataclasses.replace(w, kv_data=ref["kv_data"], ik_data=ref["ik_data"])
    say("[parity] decode after the cache write")
    dw.decode()
    torch.cuda.synchronize()
    s_ref, k_ref, o_ref, _ = _oracle_all(w2)
    serr = parity.check_scores(w2, dw.scores.cpu().numpy(), s_ref)
    k = dw.topk.cpu().numpy()
    same = parity.check_selection(w2, s_ref, k_ref, k)
    aerr = parity.check_decode_attention(w2, dw.out.float().cpu().numpy(), o_ref, same, k)
    parity.record("cache-write-fp8-then-decode", same, serr, aerr)


def test_nvfp4_cache_write_then_decode_sees_the_new_tokens():
    """The same end-to-end step with NVFP4 K/V and index keys: the write
    (data and scales of every plane, V's shared nibble bytes) and a decode
    over the written caches agree with the oracle's write and decode."""
    w, seq, pos, new = _cache_write_inputs(synth.NVFP4, synth.NVFP4, synth.BF16, synth.BF16,
                                           seed=78, spikes=False)
    keep = (seq >= 0) & (seq < w.num_seqs) & (pos < w.max_blocks * 128)
    seq, pos = seq[keep], pos[keep]
    new = {k: np.ascontiguousarray(v[keep]) for k, v in new.items()}
    ref = {k: getattr(w, k).copy() for k in ("kv_data", "kv_scales", "ik_data", "ik_scales")}
    oracle.cache_write(parity.oracle_problem(w), seq, pos, new["k"], new["v"], new["ik"],
                       w.block_table, ref["kv_data"], ref["kv_scales"], ref["ik_data"],
                       ref["ik_scales"])
    dw = parity.DeviceWorkload(w)
    msa.cache_write(dw.p, parity.dev(seq), parity.dev(pos), parity.dev(new["k"]),
                    parity.dev(new["v"]), parity.dev(new["ik"]), dw.block_table, dw.kv_data,
                    dw.kv_scales, dw.ik_data, dw.ik_scales)
    torch.cuda.synchronize()
    for name in ref:
        got = getattr(dw, name).cpu().numpy().view(np.uint8)
        assert np.array_equal(got, ref[name].view(np.uint8)), f"{name} differs after the write"
    w2 = dataclasses.replace(w, **ref)
    say("[parity] NVFP4 decode after the cache write")
    dw.decode()
    torch.cuda.synchronize()
    s_ref, k_ref, o_ref, _ = _oracle_all(w2)
    serr = parity.check_scores(w2, dw.scores.cpu().numpy(), s_ref)
    k = dw.topk.cpu().numpy()
    same = parity.check_selection(w2, s_ref, k_ref, k)
    aerr = parity.check_decode_attention(w2, dw.out.float().cpu().numpy(), o_ref, same, k)
    parity.record("cache-write-nvfp4-then-decode", same, serr, aerr)


@pytest.mark.parametrize("kv", [synth.FP8, synth.NVFP4])
@pytest.mark.parametrize("fused", [False, True])
def test_out_of_pool_entries_and_rows_past_the_table(kv, fused):
    """The header's two device-data rules against the oracle: table entries
    outside [0, P) (-1, P, -7; one of them a recent block, one sequence whose
    whole table is invalid) are empty blocks, and sequences longer than
    max_blocks * 128 (one with a query position past that too) see only the
    keys their table reaches."""
    lens = [5000, 2049, 64 * 128, 3000, 700]
    base = synth.make("pool", seed=191 + kv, seq_lens=lens, q_dtype=synth.BF16, kv_dtype=kv,
                      plant_per_seq=2)
    bt = base.block_table.copy()
    P = base.num_phys_blocks
    bt[0, 3], bt[0, 20] = -1, P
    bt[1, 16] = -7  # sequence 1's recent block
    bt[4, :] = -1   # nothing valid at all
    # sequences 2 and 3 claim more tokens than the table reaches (40 blocks)
    MB = 40
    bt = np.ascontiguousarray(bt[:, :MB])
    w = dataclasses.replace(base, max_blocks=MB, block_table=bt,
                            seq_lens=np.array([5000, 2049, 100000, 40 * 128 + 77, 700], np.int32),
                            rows_per_seq=1, q_pos=np.array([4999, 2048, 90000, 6000, 699], np.int32))
    dw, same = _run_and_check(w, fused, f"pool-{synth.DTYPE_NAMES[kv]}-{'fused' if fused else 'chain'}")
    o = dw.out.float().cpu().numpy()
    assert np.all(o[4] == 0.0) and np.all(dw.lse.cpu().numpy()[4] == -np.inf)
    assert np.all(dw.scores.cpu().numpy()[4] == -np.inf)


def test_merge_timeout_is_reported():
    """The split-K merge's failure path, forced from the host: with the
    merge told to give up at once (every kernel still runs to its end), the
    split units' outputs are NaN, the workspace is marked and
    msa_workspace_status reports it; later decodes on the marked workspace
    stay NaN; after the caller clears it, decodes are exact again.
    msa_sparse_attend clears its own workspace at every call."""
    w = synth.make("timeout", seed=93, seq_lens=[20000, 9000], q_dtype=synth.BF16,
                   kv_dtype=synth.FP8, plant_per_seq=2)
    dw = parity.DeviceWorkload(w)
    dw.decode(with_scores=False)
    torch.cuda.synchronize()
    ref = dw.out.float().clone()
    assert msa.workspace_status(dw.ws_decode) == 0
    say("[parity] forced merge timeout")
    try:
        msa.set_merge_spin_limit(-1)
        dw.decode(with_scores=False)
        assert msa.workspace_status(dw.ws_decode) == 5
        assert torch.isnan(dw.out.float()).all()
        dw.sparse_attend()
        assert msa.workspace_status(dw.ws_attend) == 5
    finally:
        msa.set_merge_spin_limit(1 << 20)
    dw.decode(with_scores=False)  # the marked workspace stays marked
    assert msa.workspace_status(dw.ws_decode) == 5
    assert torch.isnan(dw.out.float()).all()
    dw.ws_decode.zero_()
    dw.decode(with_scores=False)
    assert msa.workspace_status(dw.ws_decode) == 0
    assert torch.equal(dw.out.float(), ref)
    assert int(torch.count_nonzero(dw.ws_decode[:SPLIT_ZONE_BYTES])) == 0
    dw.sparse_attend()  # clears its workspace first
    assert msa.workspace_status(dw.ws_attend) == 0
    assert torch.isfinite(dw.out.float()).all()


# the status header and the split-K zone after it (launch.hpp: 512 (row,
# group) splits x 16 heads x (128 + 2) floats): the part of a workspace every
# call must find, and leave, zero
SPLIT_ZONE_BYTES = 256 + 512 * 16 * 130 * 4


def test_one_workspace_across_shapes():
    """msa_decode leaves the status header and the split-K zone of its
    workspace zero-filled, so one workspace (zeroed once) serves calls of
    different shapes in any order: two split-K decode shapes and a 640-row
    prefill chunk whose key-block attention keeps its lists and partials
    past the zone and leaves the header and the zone as they are."""
    R = 640
    qp = np.arange(5000 - R, 5000).astype(np.int32)
    ws_ = [synth.make("shapeA", seed=61, seq_lens=[9000, 40000, 128, 1], q_dtype=synth.BF16,
                      kv_dtype=synth.FP8, plant_per_seq=3),
           synth.make("shapeB", seed=62, seq_lens=[70000, 3000], q_dtype=synth.BF16,
                      kv_dtype=synth.FP8, num_q_heads=32, num_groups=8, top_k=8),
           synth.make("shapeC", seed=63, seq_lens=[5000], rows_per_seq=R, q_pos=qp,
                      q_dtype=synth.BF16, kv_dtype=synth.FP8, plant_per_seq=3)]
    dws = [parity.DeviceWorkload(w) for w in ws_]
    refs = []
    for dw in dws:  # each shape alone, on its own freshly zeroed workspace
        dw.decode(with_scores=False)
        torch.cuda.synchronize()
        refs.append((dw.topk.clone(), dw.out.clone()))
    shared = torch.zeros(max(int(dw.ws_decode.numel()) for dw in dws), dtype=torch.uint8,
                         device="cuda")
    assert shared.numel() > SPLIT_ZONE_BYTES
    for k in (0, 1, 2, 0, 1, 2, 2, 1, 0):
        dw = dws[k]
        say(f"[parity] shared workspace, shape {'ABC'[k]}")
        dw.ws_decode = shared
        dw.decode(with_scores=False)
        torch.cuda.synchronize()
        assert torch.equal(dw.topk, refs[k][0])
        assert torch.equal(dw.out.view(torch.uint8), refs[k][1].view(torch.uint8))
        assert int(torch.count_nonzero(shared[:SPLIT_ZONE_BYTES])) == 0


def test_empty_batch_and_errors():
    p = msa.Problem(num_seqs=0, max_blocks_per_seq=4, num_phys_blocks=4)
    z = torch.zeros(256, dtype=torch.uint8, device="cuda")
    i32 = torch.zeros(64, dtype=torch.int32, device="cuda")
    f32 = torch.zeros(64, dtype=torch.float32, device="cuda")
    msa.index_scores(p, z, z, None, i32, i32, None, f32)  # nothing to do
    # no block_scores and a workspace one float short: rejected before launch
    p1 = msa.Problem(num_seqs=4, max_blocks_per_seq=64, num_phys_blocks=4)
    need = msa.workspace_bytes(p1, msa.OP_DECODE)
    small = torch.zeros(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(msa.MsaError) as e:
        msa.decode(p1, z, z, None, z, z, None, i32, i32, None, None, i32, f32, None,
                   small[: need - 4])
    assert e.value.status == 3


@pytest.mark.parametrize("kv", [synth.FP8, synth.F32])
def test_rows_that_see_no_key(kv):
    """seq_len 0 and negative positions: -inf scores, empty selection, zero
    output, lse -inf -- the oracle's reading of an empty row."""
    lens = [0, 700, 300]
    qp = np.array([5, 0, -1, 699, 299, -7], np.int32)
    w = synth.make("empty", seed=3, seq_lens=lens, rows_per_seq=2, q_pos=qp, num_q_heads=8,
                   num_groups=4, q_dtype=synth.F32 if kv == synth.F32 else synth.BF16,
                   kv_dtype=kv, top_k=4)
    s_ref, k_ref, o_ref, l_ref = _oracle_all(w)
    dw = parity.DeviceWorkload(w)
    say(f"[parity] empty rows {synth.DTYPE_NAMES[kv]}")
    dw.decode()
    torch.cuda.synchronize()
    k = dw.topk.cpu().numpy()
    assert np.array_equal(k, k_ref)
    assert np.all(k_ref[[0, 1, 5]] == -1)
    s = dw.scores.cpu().numpy()
    assert np.all(s[[0, 1, 5]] == -np.inf)
    o = dw.out.float().cpu().numpy()
    assert np.all(o[[0, 1, 5]] == 0.0) and np.all(o_ref[[0, 1, 5]] == 0.0)
    assert np.all(dw.lse.cpu().numpy()[[0, 1, 5]] == -np.inf)
    parity.check_attention(w, o, o_ref)


@pytest.mark.parametrize("lens", [[5000, 20000, 130], [130 + 977 * i for i in range(32)]])
def test_decode_long_block_table_unfused_path(lens):
    """A block-table stride past the fused selection's LDS limit makes
    msa_decode take the three-kernel path; results follow the same rules.
    The status header and split zone are zero again afterwards: the pooled
    scores kept in the workspace lie past the zone, where they may stay."""
    w = synth.make(f"wide-{len(lens)}", seed=91, seq_lens=lens, q_dtype=synth.BF16,
                   kv_dtype=synth.FP8, max_blocks=9000, plant_per_seq=3)
    dw, _ = _run_and_check(w, fused=True, name=f"wide-table-{len(lens)}")
    assert int(torch.count_nonzero(dw.ws_decode[:SPLIT_ZONE_BYTES])) == 0
    assert dw.ws_decode.numel() > SPLIT_ZONE_BYTES


# ---------------------------------------------------------------------------
# many query rows per sequence (chunked prefill): the MFMA form of the scan
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G,H,kv", [(4, 64, synth.FP8), (8, 64, synth.FP8), (1, 16, synth.FP8),
                                    (4, 64, synth.NVFP4), (8, 64, synth.NVFP4),
                                    (1, 16, synth.NVFP4)])
def test_prefill_chunk(G, H, kv):
    """A causal chunk of R = 80 rows ending at each sequence's last key: more
    columns than one tile (G >= 4), more blocks than one block range, ragged
    lengths; FP8 and NVFP4 index keys (both on the MFMA indexer)."""
    R = 80
    lens = np.array([5000, 9003])
    qp = np.concatenate([np.arange(L - R, L) for L in lens]).astype(np.int32)
    w = synth.make(f"prefill-g{G}", seed=91 + G + 10 * kv, seq_lens=lens, rows_per_seq=R,
                   q_pos=qp, num_q_heads=H, num_groups=G, q_dtype=synth.BF16, kv_dtype=kv,
                   plant_per_seq=3)
    tag = "" if kv == synth.FP8 else "-nvfp4"
    _run_and_check(w, fused=True, name=f"prefill-g{G}{tag}")
    _run_and_check(w, fused=False, name=f"prefill-g{G}{tag}-chain")


def test_prefill_nvfp4_queries_far_outside_f16_range():
    """The NVFP4 MFMA indexer shifts each (row, group) query by its own power
    of two into f16's range: rows of a 32-row chunk with queries at 2^60,
    2^-60, a 2^30 spread inside one query, and a zero query (its blocks all
    tie at 0 and the lowest are kept)."""
    R = 32
    lens = np.array([4000])
    qp = np.arange(lens[0] - R, lens[0]).astype(np.int32)
    w = synth.make("prefill-iq-range", seed=177, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                   q_dtype=synth.BF16, kv_dtype=synth.NVFP4, plant_per_seq=2)
    iq = w.index_q.copy()
    iq[0::4] = _scale_bf16(iq[0::4], 60)
    iq[1::4] = _scale_bf16(iq[1::4], -60)
    iq[2::4, 1] = 0
    iq[3::4, :, :64] = _scale_bf16(iq[3::4, :, :64], 20)
    iq[3::4, :, 64:] = _scale_bf16(iq[3::4, :, 64:], -10)
    w = dataclasses.replace(w, index_q=iq)
    for fused in (False, True):
        _, same = _run_and_check(w, fused, "prefill-iq-range-nvfp4")
        assert same[2::4, 1].all(), "a zero query selects the lowest blocks on both sides"


@pytest.mark.parametrize("K,init,local", [(8, 2, 3), (32, 1, 4), (4, 0, 0)])
def test_prefill_chunk_selection_variants(K, init, local):
    """A causal chunk (R = 64, G = 8: 1,024 units, so the one-wave attention
    launch) with other top-k sizes and forced leading / trailing blocks: each
    row forces its own trailing blocks, through msa_decode and the chain."""
    R = 64
    lens = np.array([7000, 3001])
    qp = np.concatenate([np.arange(L - R, L) for L in lens]).astype(np.int32)
    base = synth.make(f"prefill-k{K}", seed=150 + K, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                      num_q_heads=64, num_groups=8, q_dtype=synth.BF16, kv_dtype=synth.FP8,
                      plant_per_seq=2, top_k=K)
    w = dataclasses.replace(base, init_blocks=init, local_blocks=local)
    _run_and_check(w, fused=True, name=f"prefill-k{K}-i{init}-l{local}")
    _run_and_check(w, fused=False, name=f"prefill-k{K}-i{init}-l{local}-chain")


@pytest.mark.parametrize("kv", [synth.FP8, synth.NVFP4])
def test_prefill_scattered_positions(kv):
    """Rows anywhere in the sequence, including ones that see no key or one
    key, block edges and a row past the sequence's end (clamped)."""
    qp = np.array([-1, 0, 1, 126, 127, 128, 129, 255, 256, 1000, 2047, 2048, 2049, 2900,
                   2998, 2999, 5000, 40, 300, 1700, 3, 64, 2222, 2500], np.int32)
    w = synth.make("prefill-scatter", seed=97 + kv, seq_lens=[3000], rows_per_seq=len(qp),
                   q_pos=qp, q_dtype=synth.BF16, kv_dtype=kv, plant_per_seq=2)
    _run_and_check(w, fused=True, name=f"prefill-scatter-{synth.DTYPE_NAMES[kv]}")


# ---------------------------------------------------------------------------
# chunked prefill (640+ rows per sequence): the attention grouped by key block
# ---------------------------------------------------------------------------

SCATTER_QP = [-1, 0, 1, 126, 127, 128, 129, 255, 256, 1000, 2047, 2048, 2049, 2900,
              2998, 2999, 5000, 40, 300, 1700, 3, 64, 2222, 2500]


@pytest.mark.parametrize("kv", [synth.FP8, synth.NVFP4])
def test_key_block_attention_edge_cases(kv):
    """Two sequences of 640 rows: one at scattered positions (rows that see no
    key or one key, block edges, positions past the end), one causal at its
    end; an out-of-pool table entry in each sequence, one of them the recent
    block of some rows.  Through msa_decode and the chain, then
    msa_sparse_attend on a given selection with malformed entries (-1, past
    the row's recent block, a duplicate, attended twice as by the oracle):
    outputs and lse against the oracle."""
    R = 640
    lens = np.array([3000, 4100])
    qp = np.concatenate([np.array((SCATTER_QP * 27)[:R]),
                         np.arange(lens[1] - R, lens[1])]).astype(np.int32)
    base = synth.make(f"k2q-edge-{kv}", seed=211 + kv, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                      num_q_heads=16, q_dtype=synth.BF16, kv_dtype=kv, plant_per_seq=2)
    bt = base.block_table.copy()
    bt[0, 5] = -1
    bt[1, 31] = base.num_phys_blocks  # the recent block of sequence 1's rows 3968 .. 4095
    w = dataclasses.replace(base, block_table=bt)
    tag = synth.DTYPE_NAMES[kv]
    say(f"[parity] k2q-edge-{tag}: oracle on {w.rows} rows")
    ref = _oracle_all(w)
    _run_and_check(w, fused=True, name=f"k2q-edge-{tag}", ref=ref)
    dw, _ = _run_and_check(w, fused=False, name=f"k2q-edge-{tag}-chain", ref=ref)
    # a given selection with malformed entries, inside each row's first
    # min(K, rb + 1) slots (the entries the kernels read)
    k_given = dw.topk.cpu().numpy().copy()
    for r in range(w.rows):
        rb = parity.row_pos(w, r) // w.block_size
        if rb >= 3:
            k_given[r, 0, 1] = -1
            if w.max_blocks - 1 > rb:  # a block the row does not see, inside the table
                k_given[r, 1, 0] = w.max_blocks - 1
            k_given[r, 2, 1] = k_given[r, 2, 0]
    import oracle
    o_ref, l_ref = oracle.sparse_attend(parity.oracle_problem(w), w.q, w.kv_data, w.kv_scales,
                                        w.block_table, w.seq_lens,
                                        np.ascontiguousarray(k_given, np.int32), w.q_pos)
    say(f"[parity] k2q-edge-{tag}: sparse_attend on a malformed given selection")
    dw.sparse_attend(topk=parity.dev(k_given))
    torch.cuda.synchronize()
    parity.check_attention(w, dw.out.float().cpu().numpy(), o_ref)
    lse = dw.lse.cpu().numpy()
    assert np.array_equal(np.isinf(lse), np.isinf(l_ref))
    fin = np.isfinite(l_ref)
    np.testing.assert_allclose(lse[fin], l_ref[fin], rtol=0, atol=2e-3)


def test_key_block_attention_many_chunks_per_block():
    """700 causal rows with the first block forced for every row: bucket 0
    of each group holds 700 entries, eleven work chunks; local_blocks = 2.
    Through msa_decode and the chain."""
    R = 700
    lens = np.array([20000])
    qp = np.arange(lens[0] - R, lens[0]).astype(np.int32)
    base = synth.make("k2q-chunks", seed=233, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                      num_q_heads=16, q_dtype=synth.BF16, kv_dtype=synth.FP8, plant_per_seq=3)
    w = dataclasses.replace(base, init_blocks=1, local_blocks=2)
    say(f"[parity] k2q-chunks: oracle on {w.rows} rows")
    ref = _oracle_all(w)
    dw, _ = _run_and_check(w, fused=True, name="k2q-chunks", ref=ref)
    assert np.all(dw.topk.cpu().numpy()[:, :, 0] == 0)
    _run_and_check(w, fused=False, name="k2q-chunks-chain", ref=ref)


@pytest.mark.parametrize("G,H,kv", [(8, 64, synth.NVFP4), (1, 16, synth.FP8)])
def test_key_block_attention_groups(G, H, kv):
    """640 causal rows with G = 8 (8 heads per group: half of each MFMA
    column tile is padding) over NVFP4, and G = 1 over FP8; through
    msa_decode and the chain."""
    R = 640
    lens = np.array([6000])
    qp = np.arange(lens[0] - R, lens[0]).astype(np.int32)
    w = synth.make(f"k2q-g{G}", seed=251 + G, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                   num_q_heads=H, num_groups=G, q_dtype=synth.BF16, kv_dtype=kv,
                   plant_per_seq=3)
    tag = synth.DTYPE_NAMES[kv]
    say(f"[parity] k2q-g{G}-{tag}: oracle on {w.rows} rows")
    ref = _oracle_all(w)
    _run_and_check(w, fused=True, name=f"k2q-g{G}-{tag}", ref=ref)
    _run_and_check(w, fused=False, name=f"k2q-g{G}-{tag}-chain", ref=ref)


@pytest.mark.parametrize("K,init,local,kv", [(32, 2, 3, synth.FP8), (32, 0, 0, synth.NVFP4),
                                           (4, 0, 0, synth.FP8), (1, 0, 0, synth.FP8)])
def test_key_block_attention_top_k(K, init, local, kv):
    """640 causal rows per sequence with top-k other than 16: 32 (the merge
    takes its partials in two batches of 16; count slices of 128 rows), with
    and without forced blocks, 4, and 1 (only each row's recent block, always
    the masked case).  Two sequences (G = 2, 4 heads per group), one of them
    shorter than 32 blocks (rows whose whole past is selected).  Through msa_decode and the chain,
    against one oracle run."""
    R = 640
    lens = np.array([5500, 3000])
    qp = np.concatenate([np.arange(L - R, L) for L in lens]).astype(np.int32)
    base = synth.make(f"k2q-k{K}", seed=263 + K + kv, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                      num_q_heads=8, num_groups=2, top_k=K, q_dtype=synth.BF16, kv_dtype=kv,
                      plant_per_seq=3)
    w = dataclasses.replace(base, init_blocks=init, local_blocks=local)
    tag = f"k2q-k{K}-i{init}-l{local}-{synth.DTYPE_NAMES[kv]}"
    say(f"[parity] {tag}: oracle on {w.rows} rows")
    ref = _oracle_all(w)
    _run_and_check(w, fused=True, name=tag, ref=ref)
    _run_and_check(w, fused=False, name=tag + "-chain", ref=ref)


def test_key_block_attention_1024_rows():
    """1,024 causal rows against the oracle on every row (G = 2 with 4 heads
    per group keeps the oracle small): each of the chunk's recent blocks is
    the forced block of 128 rows and spans several work chunks.  Through
    msa_decode and the chain."""
    R = 1024
    lens = np.array([4000])
    qp = np.arange(lens[0] - R, lens[0]).astype(np.int32)
    w = synth.make("k2q-1024", seed=239, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                   num_q_heads=8, num_groups=2, q_dtype=synth.BF16, kv_dtype=synth.FP8,
                   plant_per_seq=3)
    say(f"[parity] k2q-1024: oracle on {w.rows} rows")
    ref = _oracle_all(w)
    _run_and_check(w, fused=True, name="k2q-1024", ref=ref)
    _run_and_check(w, fused=False, name="k2q-1024-chain", ref=ref)


def test_key_block_attention_is_deterministic_and_equals_the_chain():
    """Which wave attends which entry follows the order of atomics; the
    results do not: repeated msa_decode calls and the three-call chain give
    bit-identical outputs and lse."""
    R = 640
    lens = np.array([9000, 6100])
    qp = np.concatenate([np.arange(L - R, L) for L in lens]).astype(np.int32)
    w = synth.make("k2q-det", seed=47, seq_lens=lens, rows_per_seq=R, q_pos=qp,
                   q_dtype=synth.BF16, kv_dtype=synth.FP8, plant_per_seq=3)
    dw = parity.DeviceWorkload(w)
    say("[parity] k2q: chain vs decode vs decode")
    dw.chain()
    torch.cuda.synchronize()
    ref = (dw.out.view(torch.uint8).clone(), dw.lse.clone(), dw.topk.clone())
    for _ in range(2):
        dw.out.zero_()
        dw.lse.zero_()
        dw.decode()
        torch.cuda.synchronize()
        assert torch.equal(dw.topk, ref[2])
        assert torch.equal(dw.out.view(torch.uint8), ref[0])
        assert torch.equal(dw.lse, ref[1])


def test_key_block_attention_8000_blocks():
    """A 640-row chunk over a 1,040,000-token context (8,125 blocks, near the
    key-block path's 8,192-block limit): each thread of the list scan takes 8
    blocks and the count's histogram spans 32 KB of LDS.  Rows at the end of
    the context plus a few far back.  The oracle on sampled rows; every row's
    selection against its own pooled scores; msa_decode equal to the chain
    bit for bit."""
    R, L = 640, 1_040_000
    qp = np.arange(L - R, L).astype(np.int32)
    qp[[5, 77, 200, 311]] = [0, 127, 128, 500_000]
    w = synth.make("k2q-8000", seed=271, seq_lens=[L], rows_per_seq=R, q_pos=qp,
                   num_q_heads=8, num_groups=2, q_dtype=synth.BF16, kv_dtype=synth.FP8,
                   plant_per_seq=6)
    assert w.max_blocks == 8125
    dw = parity.DeviceWorkload(w)
    say("[parity] k2q-8000: GPU three-call chain, then msa_decode")
    dw.chain()
    torch.cuda.synchronize()
    ref = (dw.out.view(torch.uint8).clone(), dw.lse.clone(), dw.topk.clone())
    dw.out.zero_()
    dw.decode()
    torch.cuda.synchronize()
    assert torch.equal(dw.topk, ref[2])
    assert torch.equal(dw.out.view(torch.uint8), ref[0])
    assert torch.equal(dw.lse, ref[1])
    rows = [0, 5, 77, 128, 200, 311, 383]
    ws = parity.subset_rows(w, rows)
    say(f"[parity] k2q-8000: oracle on rows {rows}")
    s_ref, k_ref, o_ref, l_ref = _oracle_all(ws)
    serr = parity.check_scores(ws, dw.scores.cpu().numpy()[rows], s_ref)
    same = parity.check_selection(ws, s_ref, k_ref, dw.topk.cpu().numpy()[rows])
    aerr = parity.check_decode_attention(ws, dw.out.float().cpu().numpy()[rows], o_ref, same,
                                         dw.topk.cpu().numpy()[rows])
    parity.record("k2q-8000 (sampled rows)", same, serr, aerr)
    S = dw.scores.cpu().numpy()
    K = dw.topk.cpu().numpy()
    assert np.isfinite(dw.out.float().cpu().numpy()).all()
    for r in range(w.rows):
        rb = parity.row_pos(w, r) // w.block_size
        for g in range(w.num_groups):
            sel = K[r, g][K[r, g] >= 0]
            if rb + 1 <= w.top_k:
                assert np.array_equal(sel, np.arange(rb + 1)), (r, g)
                continue
            cand = S[r, g, :rb]
            order = np.lexsort((np.arange(rb), -cand))[: w.top_k - 1]
            assert np.array_equal(np.sort(order), sel[:-1]) and sel[-1] == rb, (r, g)


@pytest.mark.parametrize("name", ["prefill_64k", "prefill_64k_nvfp4"])
def test_prefill_64k_sampled_rows(name):
    """The full chunked-prefill shape (65536 cached + 4096 queries, causal),
    FP8 and NVFP4, all rows on the GPU; the oracle computes a sample of rows
    one by one."""
    say(f"[parity] generating {name}")
    w = getattr(synth, name)()
    dw = parity.DeviceWorkload(w)
    say(f"[parity] {name}: GPU msa_decode over 4096 rows")
    dw.decode()
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 1000, 2047, 2048, 3333, 4094, 4095]
    ws = parity.subset_rows(w, rows)
    say(f"[parity] {name}: oracle on rows {rows}")
    s_ref, k_ref, o_ref, l_ref = _oracle_all(ws)
    s = dw.scores.cpu().numpy()[rows]
    k = dw.topk.cpu().numpy()[rows]
    o = dw.out.float().cpu().numpy()[rows]
    serr = parity.check_scores(ws, s, s_ref)
    same = parity.check_selection(ws, s_ref, k_ref, k)
    aerr = parity.check_decode_attention(ws, o, o_ref, same, k)
    parity.record(f"{name} (sampled rows)", same, serr, aerr)
    say(f"[parity] {name}: score err {serr:.3f} of bound, {int(same.sum())}/{same.size} "
        f"selections identical, attention max-abs {aerr:.2e}")
    # every row, against properties that hold at any size: the selection is
    # the top-(k-1) of the row's own pooled scores by (score desc, block asc)
    # plus its recent block, ascending; scores are -inf past the recent
    # block; outputs and lse are finite
    S = dw.scores.cpu().numpy()
    K = dw.topk.cpu().numpy()
    assert np.isfinite(dw.out.float().cpu().numpy()).all()
    assert np.isfinite(dw.lse.cpu().numpy()).all()
    for r in range(w.rows):
        rb = parity.row_pos(w, r) // w.block_size
        assert np.all(S[r, :, rb + 1:] == -np.inf)
        for g in range(w.num_groups):
            sel = K[r, g]
            assert np.all(np.diff(sel) > 0) and sel[-1] == rb
            cand = S[r, g, :rb]
            order = np.lexsort((np.arange(rb), -cand))[: w.top_k - 1]
            assert np.array_equal(np.sort(order), sel[:-1]), (r, g)
    say(f"[parity] {name}: all {w.rows} rows x {w.num_groups} groups select their own top-"
        f"{w.top_k - 1} + recent block")


# ---------------------------------------------------------------------------
# full-size workloads (the benchmark's shapes and launch configuration)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["fp8_b32", "fp8_long", "fp8_256k", "nvfp4_512k"])
def test_full_size(name):
    say(f"[parity] generating {name}")
    w = getattr(synth, name)()
    dw, same = _run_and_check(w, fused=True, name=name)
    assert same.mean() > 0.9


@pytest.mark.parametrize("name", ["fp8_share64", "nvfp4_share64"])
def test_full_size_shared_prefix(name):
    """The shared-prefix batches (64 requests on one 131,072-token prefix,
    one share group of 64): msa_decode with the share hint against the
    oracle on every output, then bit for bit against the same call without
    the hint (scores, selection, output, lse)."""
    say(f"[parity] generating {name}")
    w = getattr(synth, name)()
    assert w.share_seqs == 64
    dw, same = _run_and_check(w, fused=True, name=name)
    assert same.mean() > 0.9
    hinted = (dw.scores.clone(), dw.topk.clone(), dw.out.view(torch.uint8).clone(), dw.lse.clone())
    say(f"[parity] {name}: the same call without the share hint")
    dw0 = parity.DeviceWorkload(dataclasses.replace(w, share_seqs=0))
    dw0.decode()
    torch.cuda.synchronize()
    assert torch.equal(dw0.scores, hinted[0])
    assert torch.equal(dw0.topk, hinted[1])
    assert torch.equal(dw0.out.view(torch.uint8), hinted[2])
    assert torch.equal(dw0.lse, hinted[3])
