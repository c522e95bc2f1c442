"""Pins of the CPU oracle against facts that do not come from the oracle.

Every test here runs on the CPU.  The pins are: library decoders of the same
formats (torch's float8_e4m3fn / bfloat16), the OCP tables, exact integer
arithmetic, brute-force sorting, an independent dense-attention
implementation in torch float64, closed-form special cases, and the byte
arithmetic the pages print (tests/golden/page_numbers.txt).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.txt")


def golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("|")[0].split()
            vals[k] = float(v)
    return vals


# ---------------------------------------------------------------------------
# element formats
# ---------------------------------------------------------------------------

def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_spec_points():
    assert oracle.e4m3(0x7E) == 448.0
    assert oracle.e4m3(0xFE) == -448.0
    assert oracle.e4m3(0x08) == 2.0 ** -6
    assert oracle.e4m3(0x01) == 2.0 ** -9
    assert oracle.e4m3(0x38) == 1.0
    assert oracle.e4m3(0xC0) == -2.0
    assert len({oracle.e4m3(c) for c in range(256) if c != 0x7F and c != 0xFF}) == 253
    assert golden()["e4m3_scales"] == 256


def test_e2m1_table():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX spec, FP4 E2M1
    got = [oracle.e2m1(c) for c in range(16)]
    assert got[:8] == mags
    assert got[8:] == [-m for m in mags]
    assert len(set(abs(v) for v in got)) == golden()["e2m1_magnitudes"]


def _e4m3_test_values():
    rng = np.random.default_rng(3)
    v = np.array([oracle.e4m3(c) for c in range(0x7F)])
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)  # every tie between neighbours
    x = np.concatenate([rng.normal(0, 50, 3000), rng.normal(0, 0.01, 2000), mid, -mid,
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10]]).astype(np.float32)
    return x


def test_e4m3_encoder_matches_torch_and_the_generator():
    """Round to nearest even, every tie between neighbouring codes included:
    torch's float8_e4m3fn cast and the input generator's own encoder agree
    with the oracle's code-search encoder (within +-448, where torch does
    not saturate)."""
    x = _e4m3_test_values()
    ours = np.array([oracle.encode_e4m3(float(t)) for t in x], np.uint8)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(ours, synth.encode_e4m3(x))


def test_e4m3_encoder_saturates_and_keeps_the_sign():
    assert oracle.encode_e4m3(449.0) == 0x7E
    assert oracle.encode_e4m3(1e30) == 0x7E and oracle.encode_e4m3(-1e30) == 0xFE
    assert oracle.encode_e4m3(math.inf) == 0x7E and oracle.encode_e4m3(-math.inf) == 0xFE
    assert oracle.encode_e4m3(-1e-6) == 0x80 and oracle.encode_e4m3(-0.0) == 0x80


def test_e2m1_encoder_round_trip_ties_and_saturation():
    for c in range(16):  # every code decodes to a value that encodes back to it
        assert oracle.encode_e2m1(oracle.e2m1(c)) == c
    # the midpoints between neighbouring magnitudes go to the even code
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for c in range(7):
        m = (mags[c] + mags[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.encode_e2m1(m) == even
        assert oracle.encode_e2m1(-m) == even | 8
        assert oracle.encode_e2m1(m * (1 - 1e-9)) == c
        assert oracle.encode_e2m1(m * (1 + 1e-9)) == c + 1
    assert oracle.encode_e2m1(7.0) == 7 and oracle.encode_e2m1(-1e9) == 15


def _cache_write_case(kv, ik, q_dtype, iq_dtype, seed=5):
    """A small problem, its generated caches, and new tokens (some out of
    range) with their values."""
    lens = [900, 300, 129]
    w = synth.make("cw", seed=seed, seq_lens=lens, num_q_heads=16, num_groups=2,
                   q_dtype=q_dtype, index_q_dtype=iq_dtype, kv_dtype=kv, index_k_dtype=ik,
                   k_scale=0.75, v_scale=1.25, ik_scale=0.5 if ik != synth.NVFP4 else None)
    seq = np.array([0, 0, 0, 1, 1, 2, 2, -1, 3, 0], np.int32)
    pos = np.array([0, 1, 899, 128, 129, 127, 128, 5, 5, w.max_blocks * 128], np.int32)
    rng = np.random.default_rng(seed)
    n, G, D = len(seq), w.num_groups, w.head_dim
    vals = lambda *shape: (rng.normal(0, 2.0, shape) * np.where(rng.random(shape) < 0.1, 1e-3, 1)
                           ).astype(np.float32)
    enc = lambda x, dt: x if dt == synth.F32 else synth.encode_bf16(x)
    new = dict(k=enc(vals(n, G, D), q_dtype), v=enc(vals(n, G, D), q_dtype),
               ik=enc(vals(n, w.index_dim), iq_dtype))
    return w, seq, pos, new


def _oracle_write(w, seq, pos, new):
    caches = {k: (None if getattr(w, k) is None else getattr(w, k).copy())
              for k in ("kv_data", "kv_scales", "ik_data", "ik_scales")}
    oracle.cache_write(parity_problem(w), seq, pos, new["k"], new["v"], new["ik"],
                       w.block_table, caches["kv_data"], caches["kv_scales"],
                       caches["ik_data"], caches["ik_scales"])
    return caches


def parity_problem(w):
    return oracle.Problem(**w.problem_fields())


def test_cache_write_fp8_bytes_are_torch_casts_at_the_right_slots():
    """Each new value lands, as torch's e4m3 cast of x / scale, exactly at
    the slot the read side takes it from (K [t][d], V [d][t], index keys
    [t][d]); out-of-range tokens and every other byte are left alone."""
    w, seq, pos, new = _cache_write_case(synth.FP8, synth.FP8, synth.BF16, synth.BF16)
    c = _oracle_write(w, seq, pos, new)
    kv = w.kv_data.copy()
    ik = w.ik_data.copy()
    bf = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    cast = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i, (b, p) in enumerate(zip(seq, pos)):
        if b < 0 or b >= w.num_seqs or p >= w.max_blocks * 128:
            continue
        pb, t = w.block_table[b, p // 128], p % 128
        for g in range(w.num_groups):
            kv[pb, 0, g, t, :] = cast(np.float32(bf(new["k"][i, g])) / np.float32(w.k_scale))
            kv[pb, 1, g, :, t] = cast(np.float32(bf(new["v"][i, g])) / np.float32(w.v_scale))
        ik[pb, t, :] = cast(np.float32(bf(new["ik"][i])) / np.float32(w.index_k_scale))
    assert np.array_equal(c["kv_data"], kv)
    assert np.array_equal(c["ik_data"], ik)


def test_cache_write_nvfp4_representable_values_come_back_exactly():
    """Values built as e4m3(s) * e2m1(q) * scale, with each group holding a
    +-6 element (so amax / (6 scale) is exactly the e4m3 value of s), are
    stored as exactly those codes: the NVFP4 write is exact on its own grid."""
    import dataclasses
    w, seq, pos, new = _cache_write_case(synth.NVFP4, synth.NVFP4, synth.BF16, synth.BF16)
    w = dataclasses.replace(w, k_scale=2.0 ** -8)  # a power of two: every product exact
    rng = np.random.default_rng(9)
    G, D = w.num_groups, w.head_dim
    s_codes = rng.integers(0x20, 0x50, (len(seq), G, D // 16))
    q_codes = rng.integers(0, 16, (len(seq), G, D))
    q_codes[..., ::16] = 7  # one +6 per group
    e4 = np.vectorize(oracle.e4m3)(s_codes)
    e2 = np.vectorize(oracle.e2m1)(q_codes)
    x = (np.repeat(e4, 16, axis=-1) * e2 * w.k_scale).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), np.repeat(e4, 16, axis=-1) * e2 * w.k_scale)
    bfx = synth.encode_bf16(x)
    assert np.array_equal((bfx.astype(np.uint32) << 16).view(np.float32), x)  # bf16-exact
    new["k"] = bfx
    c = _oracle_write(w, seq, pos, new)
    b, p = int(seq[0]), int(pos[0])
    pb, t = w.block_table[b, p // 128], p % 128
    for g in range(G):
        plane = c["kv_data"][pb, 0, g].reshape(128, D // 2)[t]
        got_q = np.stack([plane & 15, plane >> 4], -1).reshape(D)
        got_q = np.where(got_q == 8, 0, got_q)  # a zero element may keep its sign
        want_q = np.where(q_codes[0, g] == 8, 0, q_codes[0, g])
        assert np.array_equal(got_q, want_q)
        sc = c["kv_scales"][pb, 0, g].reshape(128, D // 16)[t]
        assert np.array_equal(sc, s_codes[0, g])


# An independent NVFP4 writer in numpy, written from the quantiser's
# definition (per 16 consecutive elements of one token: s = e4m3(amax /
# (6 scale)), element e2m1(x / (e4m3value(s) scale)), every step one binary32
# operation, 0 codes when the group scale is 0) and the cache layouts the
# library header documents.  Rounding to e4m3 is torch's float8 cast after a
# clamp at 448 (saturation); rounding to e2m1 is a threshold table whose
# midpoints go to the even code.
def _e2m1_codes(y: np.ndarray) -> np.ndarray:
    a = np.abs(y.astype(np.float64))
    code = np.zeros(a.shape, np.uint8)
    for thr, c, inclusive in [(0.25, 1, False), (0.75, 2, True), (1.25, 3, False),
                              (1.75, 4, True), (2.5, 5, False), (3.5, 6, True),
                              (5.0, 7, False)]:
        code = np.where(a >= thr if inclusive else a > thr, np.uint8(c), code)
    return (code | (np.signbit(y).astype(np.uint8) << 3)).astype(np.uint8)


def _nvfp4_group_codes(x: np.ndarray, scale: float):
    """x [n] float32 (n a multiple of 16) -> e2m1 codes [n], e4m3 scale codes [n/16]."""
    sc = np.float32(scale)
    g = x.astype(np.float32).reshape(-1, 16)
    amax = np.abs(g).max(axis=1)
    sv = amax / (np.float32(6.0) * sc)
    s_code = torch.from_numpy(np.minimum(sv, np.float32(448.0))).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    s_val = torch.from_numpy(s_code.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    sg = (s_val * sc).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = g / sg[:, None]
    q = np.where(sg[:, None] == 0, np.uint8(0), _e2m1_codes(y))
    return q.reshape(-1), s_code


def _put_nibble(buf: np.ndarray, elem: int, code: int):
    b = elem // 2
    buf[b] = (buf[b] & 0xF0) | code if elem % 2 == 0 else (buf[b] & 0x0F) | (code << 4)


def _numpy_nvfp4_write(w, seq, pos, new):
    """Expected NVFP4 caches after writing the new tokens (both K/V and
    index keys NVFP4)."""
    P, G, BS, D, Di = w.num_phys_blocks, w.num_groups, w.block_size, w.head_dim, w.index_dim
    kvd = w.kv_data.copy().reshape(P, 2, G, -1)
    kvs = w.kv_scales.copy().reshape(P, 2, G, -1)
    ikd = w.ik_data.copy().reshape(P, BS, Di // 2)
    iks = w.ik_scales.copy().reshape(P, BS, Di // 16)
    bf = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    for i, (b, p_) in enumerate(zip(seq, pos)):
        if b < 0 or b >= w.num_seqs or p_ < 0 or p_ >= w.max_blocks * BS:
            continue
        pb = int(w.block_table[b, p_ // BS])
        if pb < 0 or pb >= P:
            continue
        t = int(p_ % BS)
        for g in range(G):
            qk, sk = _nvfp4_group_codes(bf(new["k"][i, g]), w.k_scale)
            for d in range(D):  # K: [t][d/2], scales [t][d/16]
                _put_nibble(kvd[pb, 0, g], t * D + d, int(qk[d]))
            kvs[pb, 0, g, t * (D // 16): (t + 1) * (D // 16)] = sk
            qv, sv = _nvfp4_group_codes(bf(new["v"][i, g]), w.v_scale)
            for d in range(D):  # V: [d][t/2], scales [d/16][t]
                _put_nibble(kvd[pb, 1, g], d * BS + t, int(qv[d]))
            for c in range(D // 16):
                kvs[pb, 1, g, c * BS + t] = sv[c]
        qi, si = _nvfp4_group_codes(bf(new["ik"][i]), w.index_k_scale)
        row = ikd[pb, t]
        for d in range(Di):
            _put_nibble(row, d, int(qi[d]))
        iks[pb, t] = si
    return {"kv_data": kvd.reshape(w.kv_data.shape), "kv_scales": kvs.reshape(w.kv_scales.shape),
            "ik_data": ikd.reshape(w.ik_data.shape), "ik_scales": iks.reshape(w.ik_scales.shape)}


def _nvfp4_tokens(w):
    """New tokens at block edges, both tokens of V nibble pairs (even and odd
    slot of one block), and entries out of range (skipped)."""
    seq = np.array([0, 0, 0, 0, 1, 1, 2, -1, 3, 0], np.int32)
    pos = np.array([0, 1, 898, 899, 128, 255, 127, 5, 5, w.max_blocks * 128], np.int32)
    return seq, pos


def test_cache_write_nvfp4_matches_an_independent_writer_on_every_plane():
    """General values (normal, with a spread of magnitudes, exact zeros and
    groups that are all zero): the oracle's NVFP4 K, V and index-key bytes,
    data and scales, equal those of the independent numpy writer byte for
    byte -- every plane, the transposed V with its shared nibble bytes and
    [d/16][t] scales included."""
    w, _, _, _ = _cache_write_case(synth.NVFP4, synth.NVFP4, synth.BF16, synth.BF16, seed=8)
    seq, pos = _nvfp4_tokens(w)
    rng = np.random.default_rng(17)
    n, G, D = len(seq), w.num_groups, w.head_dim

    def vals(*shape):
        x = rng.normal(0, 1.5, shape) * np.exp2(rng.integers(-12, 4, shape))
        x[rng.random(shape) < 0.05] = 0.0
        return x

    kx, vx, ix = vals(n, G, D), vals(n, G, D), vals(n, w.index_dim)
    kx[1, 0, 16:32] = 0.0  # a group with amax 0: scale code 0, data 0
    new = dict(k=synth.encode_bf16(kx), v=synth.encode_bf16(vx), ik=synth.encode_bf16(ix))
    got = _oracle_write(w, seq, pos, new)
    want = _numpy_nvfp4_write(w, seq, pos, new)
    for name in ("kv_data", "kv_scales", "ik_data", "ik_scales"):
        diff = int((got[name] != want[name]).sum())
        assert diff == 0, f"{name}: {diff} bytes differ"
    assert not np.array_equal(got["kv_data"], w.kv_data)


def test_cache_write_nvfp4_grid_values_come_back_through_an_independent_reader():
    """Values on the format's grid (e4m3(s) * e2m1(q) * scale, each group
    holding a +-6 element) for K, V and the index key, written for tokens that
    share V nibble bytes: read back with the test's own decoders of the
    documented layouts, every written element is exactly the input value and
    every element of other slots is unchanged."""
    import dataclasses
    w, _, _, _ = _cache_write_case(synth.NVFP4, synth.NVFP4, synth.BF16, synth.BF16, seed=9)
    w = dataclasses.replace(w, k_scale=2.0 ** -8, v_scale=2.0 ** -7, index_k_scale=2.0 ** -6)
    seq, pos = _nvfp4_tokens(w)
    rng = np.random.default_rng(10)
    n, G, D, Di = len(seq), w.num_groups, w.head_dim, w.index_dim

    def grid(shape, scale):
        s_codes = rng.integers(0x20, 0x50, shape[:-1] + (shape[-1] // 16,))
        q_codes = rng.integers(0, 16, shape)
        q_codes[..., ::16] = np.where(rng.random(q_codes[..., ::16].shape) < 0.5, 7, 15)
        e4 = np.vectorize(oracle.e4m3)(s_codes)
        e2 = np.vectorize(oracle.e2m1)(q_codes)
        x = np.repeat(e4, 16, axis=-1) * e2 * scale
        assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
        bx = synth.encode_bf16(x.astype(np.float32))
        assert np.array_equal((bx.astype(np.uint32) << 16).view(np.float32), x)  # bf16-exact
        return x, bx

    kx, kb = grid((n, G, D), w.k_scale)
    vx, vb = grid((n, G, D), w.v_scale)
    ix, ib = grid((n, Di), w.index_k_scale)
    got = _oracle_write(w, seq, pos, dict(k=kb, v=vb, ik=ib))
    w2 = dataclasses.replace(w, kv_data=got["kv_data"], kv_scales=got["kv_scales"],
                             ik_data=got["ik_data"], ik_scales=got["ik_scales"])
    K0, V0 = _kv_f64(w)
    K1, V1 = _kv_f64(w2)  # [P, G, BS, D], tensor scales applied
    I0 = _index_keys_f64(w) * w.index_k_scale
    I1 = _index_keys_f64(w2) * w.index_k_scale  # [P, BS, Di]
    written = set()
    for i, (b, p_) in enumerate(zip(seq, pos)):
        if b < 0 or b >= w.num_seqs or p_ >= w.max_blocks * 128:
            continue
        pb, t = int(w.block_table[b, p_ // 128]), int(p_ % 128)
        written.add((pb, t))
        for g in range(G):
            np.testing.assert_array_equal(K1[pb, g, t], kx[i, g])
            np.testing.assert_array_equal(V1[pb, g, t], vx[i, g])
        np.testing.assert_array_equal(I1[pb, t], ix[i])
    keep = np.ones((w.num_phys_blocks, 128), bool)
    for pb, t in written:
        keep[pb, t] = False
    assert np.array_equal(K1.transpose(0, 2, 1, 3)[keep], K0.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(V1.transpose(0, 2, 1, 3)[keep], V0.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(I1[keep], I0[keep])


def test_bf16_matches_torch():
    rng = np.random.default_rng(1)
    bits = np.concatenate([rng.integers(0, 1 << 16, 20000),
                           [0, 0x8000, 0x3F80, 0x7F7F, 0x0001, 0x8001]]).astype(np.int64)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------------------
# tiny problems built by hand
# ---------------------------------------------------------------------------

def _tiny_problem(B=2, G=2, hpg=2, D=16, Di=16, BS=4, K=3, lens=(9, 14), table=None,
                  q_dtype=oracle.F32, kv_dtype=oracle.F32, max_blocks=None):
    nb = [(L + BS - 1) // BS for L in lens]
    mb = max_blocks or max(nb)
    P = sum(nb) + 3
    bt = np.zeros((B, mb), np.int32)
    if table is None:
        perm = np.random.default_rng(7).permutation(P).astype(np.int32)
        off = 0
        for b in range(B):
            bt[b, : nb[b]] = perm[off: off + nb[b]]
            off += nb[b]
    else:
        bt[:] = table
    p = oracle.Problem(num_seqs=B, num_q_heads=G * hpg, num_groups=G, head_dim=D,
                       index_dim=Di, block_size=BS, top_k=K, max_blocks=mb,
                       num_phys_blocks=P, q_dtype=q_dtype, index_q_dtype=q_dtype,
                       kv_dtype=kv_dtype, index_k_dtype=kv_dtype, num_threads=3)
    return p, bt, np.asarray(lens, np.int32)


def test_index_scores_exact_integers():
    """Small-integer queries and keys: every score is an exact integer."""
    p, bt, lens = _tiny_problem()
    p.index_scale = 1.0
    p.index_k_scale = 1.0
    rng = np.random.default_rng(3)
    iq = rng.integers(-3, 4, (p.num_seqs, p.num_groups, p.index_dim)).astype(np.float32)
    ik = rng.integers(-3, 4, (p.num_phys_blocks, p.block_size, p.index_dim)).astype(np.float32)
    got = oracle.index_scores(p, iq, ik, None, bt, lens)
    for b in range(p.num_seqs):
        L = int(lens[b])
        for g in range(p.num_groups):
            for j in range(p.max_blocks):
                toks = range(j * p.block_size, min((j + 1) * p.block_size, L))
                if len(toks) == 0:
                    assert got[b, g, j] == -np.inf
                    continue
                best = None
                for t in toks:
                    pb, slot = bt[b, t // p.block_size], t % p.block_size
                    s = sum(int(iq[b, g, d]) * int(ik[pb, slot, d]) for d in range(p.index_dim))
                    best = s if best is None else max(best, s)
                assert got[b, g, j] == best


def test_index_scores_scale_is_applied():
    p, bt, lens = _tiny_problem(lens=(8, 8))
    rng = np.random.default_rng(4)
    iq = rng.integers(-3, 4, (2, 2, 16)).astype(np.float32)
    ik = rng.integers(-3, 4, (p.num_phys_blocks, 4, 16)).astype(np.float32)
    p.index_scale, p.index_k_scale = 1.0, 1.0
    base = oracle.index_scores(p, iq, ik, None, bt, lens)
    p.index_scale, p.index_k_scale = 0.25, 0.5
    scaled = oracle.index_scores(p, iq, ik, None, bt, lens)
    assert np.array_equal(scaled, (base.astype(np.float64) * 0.125).astype(np.float32))


def test_one_hot_query_reads_fp8_key_elements():
    """q = e_d gives the key element itself: pins the index-key layout and the
    e4m3 decode inside scoring."""
    p, bt, lens = _tiny_problem(lens=(8, 12), kv_dtype=oracle.FP8)
    p.index_scale = p.index_k_scale = 1.0
    rng = np.random.default_rng(5)
    ik = rng.integers(0, 256, (p.num_phys_blocks, 4, 16)).astype(np.uint8)
    ik[ik == 0x7F] = 0x10
    ik[ik == 0xFF] = 0x90
    keys = torch.from_numpy(ik).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for d in (0, 5, 15):
        iq = np.zeros((2, 2, 16), np.float32)
        iq[:, :, d] = 1.0
        got = oracle.index_scores(p, iq, ik, None, bt, lens)
        for b in range(2):
            L = int(lens[b])
            for j in range((L + 3) // 4):
                vals = [keys[bt[b, j], t % 4, d] for t in range(j * 4, min(j * 4 + 4, L))]
                assert got[b, 0, j] == np.float32(max(vals))


def _decode_plain(arr, dtype):
    if dtype == oracle.F32:
        return arr.astype(np.float64)
    if dtype == oracle.BF16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    if dtype == oracle.FP8:
        return torch.from_numpy(arr).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    raise ValueError(dtype)


def _decode_nvfp4(data, scales):
    """data[..., n/2], scales[..., n/16] -> values[..., n] (no tensor scale)."""
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
    codes = np.stack([data & 15, data >> 4], axis=-1).reshape(data.shape[:-1] + (-1,))
    vals = table[codes]
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    return vals * np.repeat(sc, 16, axis=-1)


def _small_workload(kv_dtype, lens=(300, 517, 129), G=2, H=4, top_k=3, q_pos=None,
                    rows_per_seq=1, seed=11, plant=0):
    q_dtype = synth.F32 if kv_dtype == synth.F32 else synth.BF16
    return synth.make("t", seed=seed, seq_lens=list(lens), num_q_heads=H, num_groups=G,
                      top_k=top_k, q_dtype=q_dtype, kv_dtype=kv_dtype, q_pos=q_pos,
                      rows_per_seq=rows_per_seq, plant_per_seq=plant)


def _oracle_problem(w, threads=4):
    return oracle.Problem(**w.problem_fields(), num_threads=threads)


def _index_keys_f64(w):
    if w.index_k_dtype == synth.NVFP4:
        return _decode_nvfp4(w.ik_data, w.ik_scales)
    return _decode_plain(w.ik_data, w.index_k_dtype)


@pytest.mark.parametrize("dtype", [synth.F32, synth.FP8, synth.NVFP4])
def test_pooled_scores_brute_force(dtype):
    """Token scores by a float64 matrix product on independently decoded keys,
    rounded to fp32 and max-pooled per block (at most 1 fp32 ulp apart: only
    the double summation order differs)."""
    w = _small_workload(dtype)
    p = _oracle_problem(w)
    got = oracle.index_scores(p, w.index_q, w.ik_data, w.ik_scales, w.block_table, w.seq_lens)
    keys = _index_keys_f64(w) * w.index_k_scale  # [P, BS, Di]
    iq = _decode_plain(w.index_q, w.index_q_dtype)
    BS = w.block_size
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        nb = (L + BS - 1) // BS
        seq_keys = keys[w.block_table[b, :nb]].reshape(nb * BS, -1)[:L]
        s = (seq_keys @ iq[b].T * w.index_scale).astype(np.float32)  # [L, G]
        for j in range(w.max_blocks):
            if j >= nb:
                assert np.all(got[b, :, j] == -np.inf)
                continue
            ref = s[j * BS: min(L, (j + 1) * BS)].max(axis=0)
            np.testing.assert_array_max_ulp(got[b, :, j], ref, maxulp=1)


def test_partial_block_ignores_tokens_past_the_end():
    p, bt, lens = _tiny_problem(lens=(9, 14))
    p.index_scale = p.index_k_scale = 1.0
    iq = np.ones((2, 2, 16), np.float32)
    ik = np.zeros((p.num_phys_blocks, 4, 16), np.float32)
    # garbage in the unused slots of each sequence's last block
    for b, L in enumerate(lens):
        last = (L - 1) // 4
        ik[bt[b, last], L % 4 or 4:] = 1000.0
    got = oracle.index_scores(p, iq, ik, None, bt, lens)
    assert np.all(got[:, :, :4][np.isfinite(got[:, :, :4])] == 0.0)


def test_q_pos_limits_visible_tokens():
    """With explicit positions a row sees keys t <= pos only."""
    p, bt, lens = _tiny_problem(lens=(16, 16), K=2)
    p.rows_per_seq = 2
    p.index_scale = p.index_k_scale = 1.0
    iq = np.ones((4, 2, 16), np.float32)
    ik = np.zeros((p.num_phys_blocks, 4, 16), np.float32)
    ik[bt[0, 3], 3] = 5.0  # token 15 of seq 0
    qp = np.array([14, 15, 6, 15], np.int32)
    got = oracle.index_scores(p, iq, ik, None, bt, lens, q_pos=qp)
    assert got[0, 0, 3] == 0.0 and got[1, 0, 3] == 80.0
    assert np.all(got[2, :, 2:] == -np.inf) and np.isfinite(got[2, 0, 1])


# ---------------------------------------------------------------------------
# rows longer than their block table; table entries outside the pool (the
# readings the library header documents: a row sees only keys its table
# reaches, and an entry outside [0, P) is an empty block)
# ---------------------------------------------------------------------------

def test_rows_are_clamped_at_the_table_reach():
    """Sequences longer than max_blocks * BS, and a query position past it,
    see the keys t < max_blocks * BS only: every output equals that of the
    same caches with the lengths cut to the table's reach, and the cut case
    matches the brute-force scores and the dense attention."""
    import dataclasses
    base = _small_workload(synth.FP8, lens=(700, 517, 129), top_k=3, plant=1)
    MB = 4  # reach: 512 tokens
    bt = np.ascontiguousarray(base.block_table[:, :MB])
    cut = dataclasses.replace(base, max_blocks=MB, block_table=bt,
                              seq_lens=np.array([512, 512, 129], np.int32))
    long_ = dataclasses.replace(cut, seq_lens=np.array([700, 10517, 129], np.int32))
    a = oracle.decode(_oracle_problem(long_), long_.index_q, long_.ik_data, long_.ik_scales,
                      long_.q, long_.kv_data, long_.kv_scales, long_.block_table,
                      long_.seq_lens)
    c = oracle.decode(_oracle_problem(cut), cut.index_q, cut.ik_data, cut.ik_scales, cut.q,
                      cut.kv_data, cut.kv_scales, cut.block_table, cut.seq_lens)
    for x, y in zip(a, c):
        assert np.array_equal(x, y)
    keys = _index_keys_f64(cut) * cut.index_k_scale
    iq = _decode_plain(cut.index_q, cut.index_q_dtype)
    for b in range(cut.num_seqs):
        L = int(cut.seq_lens[b])
        nb = (L + 127) // 128
        s = (keys[cut.block_table[b, :nb]].reshape(nb * 128, -1)[:L] @ iq[b].T
             * cut.index_scale).astype(np.float32)
        for j in range(nb):
            np.testing.assert_array_max_ulp(c[0][b, :, j], s[j * 128: (j + 1) * 128].max(0), 1)
        assert all((c[1][b, g] >= 0).sum() == min(3, nb) and nb - 1 in c[1][b, g]
                   for g in range(cut.num_groups))
        ref = _dense_attention(cut, b, [[j for j in c[1][b, g] if j >= 0]
                                        for g in range(cut.num_groups)])
        np.testing.assert_allclose(c[2][b], ref, rtol=1e-12, atol=1e-12)
    # positions past the reach clamp the same way
    qp = np.array([5000, 300, 128], np.int32)
    qpc = np.array([511, 300, 128], np.int32)
    pa = oracle.decode(_oracle_problem(long_), long_.index_q, long_.ik_data, long_.ik_scales,
                       long_.q, long_.kv_data, long_.kv_scales, long_.block_table,
                       long_.seq_lens, qp)
    pc = oracle.decode(_oracle_problem(cut), cut.index_q, cut.ik_data, cut.ik_scales, cut.q,
                       cut.kv_data, cut.kv_scales, cut.block_table, cut.seq_lens, qpc)
    for x, y in zip(pa, pc):
        assert np.array_equal(x, y)


def test_out_of_pool_table_entries_are_empty_blocks():
    """Entries -1, P and -5 (one of them a recent block) score -inf, are
    never dereferenced and add nothing to the attention; a sequence whose
    whole table is invalid gets -inf scores, the plain selection, a zero
    output and lse -inf."""
    import dataclasses
    w = _small_workload(synth.FP8, lens=(900, 517, 300), top_k=4, plant=2)
    p = _oracle_problem(w)
    s0 = oracle.index_scores(p, w.index_q, w.ik_data, w.ik_scales, w.block_table, w.seq_lens)
    bt = w.block_table.copy()
    bad = {(0, 2): -1, (0, 6): w.num_phys_blocks, (1, 4): -5}  # (1, 4): sequence 1's recent block
    for (b, j), v in bad.items():
        bt[b, j] = v
    bt[2, :] = -1
    wb = dataclasses.replace(w, block_table=bt)
    s, k, o, lse = oracle.decode(p, wb.index_q, wb.ik_data, wb.ik_scales, wb.q, wb.kv_data,
                                 wb.kv_scales, bt, wb.seq_lens)
    for b in range(2):
        for j in range(w.max_blocks):
            if (b, j) in bad:
                assert np.all(s[b, :, j] == -np.inf)
            else:
                assert np.array_equal(s[b, :, j], s0[b, :, j])
    assert np.all(s[2] == -np.inf)
    for b in range(3):
        recent = (int(w.seq_lens[b]) - 1) // 128
        for g in range(w.num_groups):
            assert list(k[b, g]) == _brute_select(s[b, g], recent, w.top_k)
    valid = lambda b, j: j >= 0 and (b, j) not in bad
    for b in range(2):
        ref = _dense_attention(w, b, [[j for j in k[b, g] if valid(b, j)]
                                      for g in range(w.num_groups)])
        np.testing.assert_allclose(o[b], ref, rtol=1e-12, atol=1e-12)
    assert np.all(o[2] == 0.0) and np.all(lse[2] == -np.inf)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _brute_select(scores, recent, K):
    if recent + 1 <= K:
        sel = list(range(recent + 1))
    else:
        order = sorted(range(recent), key=lambda j: (-float(scores[j]), j))
        sel = sorted(order[: K - 1] + [recent])
    return sel + [-1] * (K - len(sel))


@pytest.mark.parametrize("K", [1, 4, 16, 32])
def test_topk_matches_brute_force_sort_with_ties(K):
    rng = np.random.default_rng(K)
    B, G, mb, BS = 6, 3, 70, 4
    lens = rng.integers(1, mb * BS + 1, B).astype(np.int32)
    lens[0] = mb * BS
    lens[1] = 1
    p = oracle.Problem(num_seqs=B, num_q_heads=G, num_groups=G, head_dim=16, index_dim=16,
                       block_size=BS, top_k=K, max_blocks=mb, num_phys_blocks=1)
    # coarse values so that many scores tie exactly
    scores = rng.integers(-4, 5, (B, G, mb)).astype(np.float32) * 0.5
    got = oracle.block_topk(p, scores, lens)
    for b in range(B):
        recent = (int(lens[b]) - 1) // BS
        for g in range(G):
            assert list(got[b, g]) == _brute_select(scores[b, g], recent, K)


def test_topk_invariants_and_recent_forced():
    rng = np.random.default_rng(2)
    B, G, mb, BS, K = 5, 4, 300, 128, 16
    lens = rng.integers(1, mb * BS + 1, B).astype(np.int32)
    p = oracle.Problem(num_seqs=B, num_q_heads=64, num_groups=G, block_size=BS, top_k=K,
                       max_blocks=mb, num_phys_blocks=1)
    scores = rng.standard_normal((B, G, mb)).astype(np.float32)
    # the recent block gets the worst score on purpose
    for b in range(B):
        scores[b, :, (lens[b] - 1) // BS] = -1e30
    got = oracle.block_topk(p, scores, lens)
    for b in range(B):
        r = (int(lens[b]) - 1) // BS
        for g in range(G):
            sel = [j for j in got[b, g] if j >= 0]
            assert len(sel) == min(K, r + 1)
            assert r in sel
            assert sel == sorted(sel) and len(set(sel)) == len(sel)
            assert all(x == -1 for x in got[b, g][len(sel):])
            assert len(sel) * BS <= golden()["max_keys_per_query"]
            others = [j for j in sel if j != r]
            if others:
                weakest = min(scores[b, g, j] for j in others)
                unsel = [j for j in range(r) if j not in sel]
                assert all(scores[b, g, j] <= weakest for j in unsel)


def _forced_set(recent, init, local):
    n_local = max(local, 1)
    return {j for j in range(recent + 1) if j < init or j > recent - n_local}


def _rank_select(scores, recent, K, init, local):
    """The selection by ranks: a free block is kept when fewer than
    (K - forced) free blocks beat it (higher score, or equal score and lower
    index)."""
    if recent + 1 <= K:
        sel = list(range(recent + 1))
    else:
        forced = _forced_set(recent, init, local)
        free = [j for j in range(recent + 1) if j not in forced]
        need = K - len(forced)
        sel = sorted(forced)
        for j in free:
            beaten_by = sum(1 for i in free
                            if scores[i] > scores[j] or (scores[i] == scores[j] and i < j))
            if beaten_by < need:
                sel.append(j)
        sel.sort()
    return sel + [-1] * (K - len(sel))


def _subset_select(scores, recent, K, init, local):
    """The selection as the best K-subset: among all K-subsets of 0..recent
    that hold the forced blocks, the one whose free members, listed best
    first as (score, -index), form the largest sequence."""
    import itertools
    if recent + 1 <= K:
        return list(range(recent + 1)) + [-1] * (K - recent - 1)
    forced = _forced_set(recent, init, local)
    free = [j for j in range(recent + 1) if j not in forced]
    best, best_key = None, None
    for comb in itertools.combinations(free, K - len(forced)):
        key = sorted(((float(scores[j]), -j) for j in comb), reverse=True)
        if best_key is None or key > best_key:
            best, best_key = comb, key
    return sorted(list(forced) + list(best))


@pytest.mark.parametrize("K,init,local", [(4, 1, 0), (4, 0, 3), (4, 2, 2), (5, 1, 2),
                                          (3, 2, 0), (3, 0, 0), (2, 0, 2)])
def test_topk_forced_blocks_match_best_subset_on_tiny_rows(K, init, local):
    rng = np.random.default_rng(100 * K + 10 * init + local)
    B, G, mb, BS = 9, 2, 11, 2
    lens = np.arange(1, B + 1, dtype=np.int32) * 2 + 3  # 2 .. 10 visible blocks
    p = oracle.Problem(num_seqs=B, num_q_heads=G, num_groups=G, head_dim=16, index_dim=16,
                       block_size=BS, top_k=K, max_blocks=mb, num_phys_blocks=1,
                       init_blocks=init, local_blocks=local)
    scores = rng.integers(-2, 3, (B, G, mb)).astype(np.float32)  # many exact ties
    got = oracle.block_topk(p, scores, lens)
    for b in range(B):
        recent = (int(lens[b]) - 1) // BS
        for g in range(G):
            want = _subset_select(scores[b, g], recent, K, init, local)
            assert [j for j in got[b, g] if j >= 0] == [j for j in want if j >= 0]


@pytest.mark.parametrize("K,init,local", [(4, 1, 1), (8, 2, 4), (16, 1, 3), (16, 8, 8),
                                          (32, 4, 0), (32, 0, 32), (8, 7, 0)])
def test_topk_forced_blocks_match_rank_rule(K, init, local):
    rng = np.random.default_rng(K + 7 * init + 31 * local)
    B, G, mb, BS = 7, 3, 90, 4
    lens = rng.integers(1, mb * BS + 1, B).astype(np.int32)
    lens[0], lens[1], lens[2] = mb * BS, 1, K * BS + 1  # full, one key, one block past k
    p = oracle.Problem(num_seqs=B, num_q_heads=G, num_groups=G, head_dim=16, index_dim=16,
                       block_size=BS, top_k=K, max_blocks=mb, num_phys_blocks=1,
                       init_blocks=init, local_blocks=local)
    scores = rng.integers(-3, 4, (B, G, mb)).astype(np.float32) * 0.25
    got = oracle.block_topk(p, scores, lens)
    for b in range(B):
        recent = (int(lens[b]) - 1) // BS
        for g in range(G):
            sel = [j for j in got[b, g] if j >= 0]
            assert list(got[b, g]) == _rank_select(scores[b, g], recent, K, init, local)
            assert len(sel) == min(K, recent + 1)
            if recent + 1 > K:
                assert _forced_set(recent, init, local) <= set(sel)


def test_topk_forced_blocks_win_over_any_score():
    """Forced blocks stay even with the worst scores; with init + local = k
    nothing else is chosen; local 0 and 1 and init 0 give the plain rule."""
    rng = np.random.default_rng(5)
    B, G, mb, BS, K = 4, 2, 200, 128, 16
    lens = np.array([mb * BS, 150 * BS + 3, 40 * BS, 17 * BS], np.int32)
    scores = rng.standard_normal((B, G, mb)).astype(np.float32)
    scores[:, :, :3] = -1e30
    for b in range(B):
        r = (int(lens[b]) - 1) // BS
        scores[b, :, r - 5:r + 1] = -1e30

    def run(init, local):
        p = oracle.Problem(num_seqs=B, num_q_heads=64, num_groups=G, block_size=BS, top_k=K,
                           max_blocks=mb, num_phys_blocks=1, init_blocks=init,
                           local_blocks=local)
        return oracle.block_topk(p, scores, lens)

    plain = run(0, 0)
    assert np.array_equal(run(0, 1), plain)
    for b in range(B):
        r = (int(lens[b]) - 1) // BS
        for g in range(G):
            assert list(plain[b, g]) == _brute_select(scores[b, g], r, K)
    got = run(3, 6)
    full = run(10, 6)
    for b in range(B):
        r = (int(lens[b]) - 1) // BS
        for g in range(G):
            sel = set(got[b, g]) - {-1}
            assert {0, 1, 2} | set(range(r - 5, r + 1)) <= sel
            assert list(full[b, g]) == list(range(10)) + list(range(r - 5, r + 1))
    with pytest.raises(ValueError):
        run(11, 6)  # 17 forced blocks do not fit in k = 16
    with pytest.raises(ValueError):
        run(16, 0)  # the recent block needs a place too


def test_topk_shard_merge_is_exact():
    """Context sharding of the indexer: each shard's local top-(k-1)
    candidates, merged, give exactly the single-device selection (vLLM blog,
    "NVFP4 indexer DCP": the owner merges the local top-16 lists and the
    selection stays exact)."""
    rng = np.random.default_rng(9)
    B, G, mb, BS, K = 3, 4, 257, 128, 16
    lens = np.array([mb * BS, 200 * BS + 5, 17 * BS], np.int32)
    p = oracle.Problem(num_seqs=B, num_q_heads=64, num_groups=G, block_size=BS, top_k=K,
                       max_blocks=mb, num_phys_blocks=1)
    scores = rng.integers(-50, 50, (B, G, mb)).astype(np.float32)  # ties across shards
    full = oracle.block_topk(p, scores, lens)
    for nshard in (2, 3, 4):
        for b in range(B):
            r = (int(lens[b]) - 1) // BS
            for g in range(G):
                cands = []
                bounds = np.linspace(0, r, nshard + 1).astype(int)
                for s in range(nshard):
                    lo, hi = bounds[s], bounds[s + 1]
                    sub = np.full((1, 1, mb), -np.inf, np.float32)
                    sub[0, 0, lo:hi] = scores[b, g, lo:hi]
                    sub[0, 0, r] = 0.0
                    p1 = oracle.Problem(num_seqs=1, num_q_heads=1, num_groups=1,
                                        block_size=BS, top_k=K, max_blocks=mb,
                                        num_phys_blocks=1)
                    loc = oracle.block_topk(p1, sub, np.array([lens[b]], np.int32))
                    cands += [j for j in loc[0, 0] if j >= 0 and lo <= j < hi]
                merged = sorted(cands, key=lambda j: (-float(scores[b, g, j]), j))
                want = sorted(merged[: K - 1] + [r]) if r + 1 > K else list(range(r + 1))
                assert [j for j in full[b, g] if j >= 0] == want


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _kv_f64(w):
    """Independent decode of the K/V pool -> K[P, G, BS, D], V[P, G, BS, D]."""
    P, G, BS, D = w.num_phys_blocks, w.num_groups, w.block_size, w.head_dim
    if w.kv_dtype == synth.NVFP4:
        kd = w.kv_data[:, 0].reshape(P, G, BS, D // 2)
        ks = w.kv_scales[:, 0].reshape(P, G, BS, D // 16)
        K = _decode_nvfp4(kd, ks)
        vd = w.kv_data[:, 1].reshape(P, G, D, BS // 2)
        vs = w.kv_scales[:, 1].reshape(P, G, D // 16, BS)
        codes = np.stack([vd & 15, vd >> 4], axis=-1).reshape(P, G, D, BS)
        table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
        sc = torch.from_numpy(np.ascontiguousarray(vs)).view(torch.float8_e4m3fn).to(
            torch.float64).numpy()
        V = np.swapaxes(table[codes] * np.repeat(sc, 16, axis=2), -1, -2)
    else:
        x = _decode_plain(w.kv_data, w.kv_dtype)
        K = x[:, 0]
        V = np.swapaxes(x[:, 1], -1, -2)
    return K * w.k_scale, V * w.v_scale


def _dense_attention(w, row, blocks):
    """softmax attention in torch float64 over the given logical blocks."""
    K, V = _kv_f64(w)
    b = row // w.rows_per_seq
    L = int(w.seq_lens[b])
    pos = int(w.q_pos[row]) if w.q_pos is not None else L - 1
    q = torch.from_numpy(_decode_plain(w.q, w.q_dtype)[row])  # [H, D]
    hpg = w.num_q_heads // w.num_groups
    out = torch.empty(w.num_q_heads, w.head_dim, dtype=torch.float64)
    for g in range(w.num_groups):
        toks = [(j, t) for j in blocks[g] for t in range(w.block_size)
                if j * w.block_size + t <= pos]
        Kg = torch.from_numpy(np.stack([K[w.block_table[b, j], g, t] for j, t in toks]))
        Vg = torch.from_numpy(np.stack([V[w.block_table[b, j], g, t] for j, t in toks]))
        qg = q[g * hpg:(g + 1) * hpg]
        att = torch.softmax(qg @ Kg.T * w.sm_scale, dim=-1)
        out[g * hpg:(g + 1) * hpg] = att @ Vg
    return out.numpy()


@pytest.mark.parametrize("dtype", [synth.F32, synth.FP8, synth.NVFP4])
def test_attend_equals_dense_when_topk_covers_everything(dtype):
    w = _small_workload(dtype, lens=(300, 517, 129), top_k=8)
    p = _oracle_problem(w)
    _, topk, out, _ = oracle.decode(p, w.index_q, w.ik_data, w.ik_scales, w.q, w.kv_data,
                                    w.kv_scales, w.block_table, w.seq_lens)
    for row in range(w.rows):
        nb = (int(w.seq_lens[row]) + 127) // 128
        assert all(list(topk[row, g][:nb]) == list(range(nb)) for g in range(w.num_groups))
        ref = _dense_attention(w, row, [list(range(nb))] * w.num_groups)
        np.testing.assert_allclose(out[row], ref, rtol=1e-12, atol=1e-12)


def test_attend_matches_dense_on_the_selected_blocks():
    w = _small_workload(synth.FP8, lens=(2000, 1500), top_k=4, plant=2)
    p = _oracle_problem(w)
    _, topk, out, lse = oracle.decode(p, w.index_q, w.ik_data, w.ik_scales, w.q, w.kv_data,
                                      w.kv_scales, w.block_table, w.seq_lens)
    for row in range(w.rows):
        blocks = [[j for j in topk[row, g] if j >= 0] for g in range(w.num_groups)]
        ref = _dense_attention(w, row, blocks)
        np.testing.assert_allclose(out[row], ref, rtol=1e-12, atol=1e-12)


def test_attend_special_cases():
    p, bt, lens = _tiny_problem(lens=(1, 14), K=2)
    rng = np.random.default_rng(12)
    H, D, P = p.num_q_heads, p.head_dim, p.num_phys_blocks
    kv = rng.standard_normal((P, 2, p.num_groups, 4, D)).astype(np.float32)
    q = rng.standard_normal((2, H, D)).astype(np.float32)
    topk = np.array([[[0, -1], [0, -1]], [[1, 3], [0, 3]]], np.int32)
    # single visible token: output is that token's v
    out, lse = oracle.sparse_attend(p, q, kv, None, bt, lens, topk)
    for g in range(2):
        v0 = kv[bt[0, 0], 1, g].reshape(D, 4)[:, 0]  # V stored [d][t]: column t=0
        for h in range(g * 2, g * 2 + 2):
            np.testing.assert_array_equal(out[0, h], v0.astype(np.float64))
    # V constant: output is that constant
    kv_c = kv.copy()
    kv_c[:, 1] = 0.375
    out_c, _ = oracle.sparse_attend(p, q, kv_c, None, bt, lens, topk)
    np.testing.assert_allclose(out_c, 0.375, rtol=0, atol=1e-15)
    # q = 0: uniform weights, mean of V over the selected visible tokens
    out0, lse0 = oracle.sparse_attend(p, np.zeros_like(q), kv, None, bt, lens, topk)
    for g in range(2):
        toks = [(j, t) for j in topk[1, g] for t in range(4) if j * 4 + t < 14]
        mean = np.mean([kv[bt[1, j], 1, g].reshape(D, 4)[:, t].astype(np.float64)
                        for j, t in toks], axis=0)
        np.testing.assert_allclose(out0[1, 2 * g], mean, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse0[1, 2 * g], math.log(len(toks)), rtol=1e-14)


def test_planted_blocks_are_selected():
    """The long-context recipe plants 8 blocks per sequence; their pooled
    score lift is large enough that every group keeps them."""
    w = _small_workload(synth.FP8, lens=(40 * 128, 33 * 128 + 7), G=4, H=8, top_k=16,
                        plant=8)
    p = _oracle_problem(w)
    scores = oracle.index_scores(p, w.index_q, w.ik_data, w.ik_scales, w.block_table,
                                 w.seq_lens)
    topk = oracle.block_topk(p, scores, w.seq_lens)
    for b, blocks in w.planted.items():
        for g in range(w.num_groups):
            assert set(blocks) <= set(topk[b, g].tolist())


# ---------------------------------------------------------------------------
# the pages' byte arithmetic
# ---------------------------------------------------------------------------

def test_page_byte_arithmetic():
    gv = golden()
    assert gv["topk_blocks"] * gv["block_size_tokens"] == gv["max_keys_per_query"]
    assert gv["fp8_kv_heads"] * gv["head_dim"] * 2 * 1 == gv["fp8_kv_bytes_per_token"]
    assert gv["index_key_bytes_per_token"] / gv["fp8_kv_bytes_per_token"] == \
        gv["index_over_dense_fraction"]
    # NVFP4 = 4-bit values + one 8-bit scale per 16 elements = 4.5 bits vs 8
    nv_bits = 4 + 8 / gv["nvfp4_group"]
    assert nv_bits / 8 == gv["nvfp4_kv_bytes_per_token_model"] / gv["fp8_kv_bytes_per_token_model"]
    assert 1 - nv_bits / 8 == gv["nvfp4_saving_fraction"]


@pytest.mark.parametrize("dtype,ik_bytes,kv_bytes", [(synth.FP8, 128, 1024),
                                                     (synth.NVFP4, 72, 576)])
def test_generated_caches_have_the_pages_bytes_per_token(dtype, ik_bytes, kv_bytes):
    w = _small_workload(dtype, lens=(256,), G=4, H=8)
    tok = w.num_phys_blocks * w.block_size
    ikb = w.ik_data.nbytes + (w.ik_scales.nbytes if w.ik_scales is not None else 0)
    kvb = w.kv_data.nbytes + (w.kv_scales.nbytes if w.kv_scales is not None else 0)
    assert ikb / tok == ik_bytes and kvb / tok == kv_bytes
    if dtype == synth.FP8:
        assert ik_bytes == golden()["index_key_bytes_per_token"]
        assert kv_bytes == golden()["fp8_kv_bytes_per_token"]
    else:
        assert kv_bytes / 1024 == golden()["nvfp4_kv_bytes_per_token_model"] / \
            golden()["fp8_kv_bytes_per_token_model"]


def test_threads_do_not_change_results():
    w = _small_workload(synth.FP8, lens=(700, 900, 1100), top_k=4)
    res = []
    for th in (1, 5):
        p = _oracle_problem(w, threads=th)
        res.append(oracle.decode(p, w.index_q, w.ik_data, w.ik_scales, w.q, w.kv_data,
                                 w.kv_scales, w.block_table, w.seq_lens))
        assert oracle.threads_used() == min(th, w.rows * w.num_groups)
    for a, b in zip(*res):
        assert np.array_equal(a, b)
