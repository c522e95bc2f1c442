// index_block.hpp -- one wavefront scores one logical block for the index
// queries of one or a few rows of a sequence.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer"): every cached key is scored by one index query per GQA group
// against one shared index-key head; the scores are max-pooled to one score
// per 128-token block.
//
// A wave takes a block in two halves of 64 tokens; each load instruction of
// the wave reads 1 KB of consecutive bytes (NVFP4 scales: 128 bytes), and a
// half's loads are all issued before its arithmetic.
//
// Arithmetic: keys are converted exactly to bf16 (e4m3 and e2m1 x e4m3 values
// are bf16-representable) and multiplied with the bf16 index queries on MFMA:
// exact products, fp32 accumulation.  The positive score scale commutes with
// the max, so it is applied once per block.
#pragma once

#include "device.hpp"
#include "launch.hpp"

namespace msa {

struct IndexArgs {
  const uint16_t* iq;  // [rows][G][128] bf16 index queries
  const uint8_t* ikd;  // index-key data, [P][128][128] e4m3 or [P][128][64] E2M1
  const uint8_t* iks;  // NVFP4: [P][128][8] e4m3 scales; otherwise unused
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* qpos;
  float* scores;  // [rows][G][MB]
  int R, G, MB, P;
  int rows_per_wave;  // rows of one sequence a wave scores together (rows_per_wave * G <= 16)
  int row_groups;     // ceil(R / rows_per_wave)
  int B;              // sequences
  int share;          // shared scan: sequences per share group (R == 1)
  float out_scale;    // index_scale * index_k_scale (NVFP4: times the tensor scale)
};

// The scores of a 16-token tile come from MFMA: S = K Q^T as
// v_mfma_f32_16x16x32_bf16 with the tile's tokens as A rows, the wave's
// index queries as B columns -- the G groups of up to 16 / G rows of one
// sequence (several rows per sequence: speculative decode), padded to 16
// with zeros -- and 4 K-chunks of 32 dims.  One pass over the keys serves
// all those rows.
// A lane's A rows are tokens lane%16 -- 16 different rows -- while the loads
// that stream HBM best read contiguous kilobytes, so a wave loads half a
// block contiguously into registers, writes it to its own LDS area, and
// reads it back in MFMA order.  The LDS rows are swizzled (16-byte chunk c
// of token t at chunk slot c ^ f(t)) so that both the writes and the reads
// are free of bank conflicts.
//
// The contraction order is free as long as A and B agree, so each format
// assigns the dims of chunk c to lane group r = lane/16 as it suits the LDS
// reads:
//   FP8  : lane reads dims [16r + 64h, +16) of its token (h = 0, 1); chunk
//          c = 2h + e takes dims 16r + 64h + 8e + 0..7;
//   NVFP4: lane reads dims [32r, +32) (16 bytes) and the two scales of
//          them; chunk e takes dims 32r + 8e + 0..7.
// D lane l holds tokens 4r + i (i = 0..3) of the tile for column l%16; a
// running max per lane over the tiles (keys up to that column's row's last
// visible key), then over i and over the four lane groups, gives the block's
// score of column l%16 (lanes 0..cols-1 keep them).

// LDS per wave: half a block staged (FP8 8 KB; NVFP4 4 KB of data plus the
// block's 1 KB of scales)
template <int IK>
constexpr int stage_bytes() {
  return IK == kFP8 ? 8192 : 5120;
}

// B operand: the wave's cols index queries, (row, group) pairs col0 ..
// col0 + cols - 1 (zero columns past cols).  FP8 keys take them as bf16.
// NVFP4 keys are dequantised to f16 (cheaper than bf16: the block scale is
// one packed f16 multiply per two values), so the queries go to f16 too,
// each column shifted by a power of two 2^sh that puts its largest element
// in [2^15, 2^16): every element within 2^32 of the column's largest then
// converts exactly, and unscale = 2^-sh undoes the shift on the pooled
// score (max-pooling commutes with a positive scale, and a power-of-two
// scale is exact).
template <int IK>
struct QueryB;
template <>
struct QueryB<kFP8> {
  bf16x8 b[4];
  float unscale;
};
template <>
struct QueryB<kNVFP4> {
  f16x8 b[4];
  float unscale;
};

__device__ __forceinline__ void load_query_b(const IndexArgs& x, size_t col0, int cols, int lane,
                                             QueryB<kFP8>& q) {
  // loads from a clamped column, masked to zero past cols (no branch, so
  // nothing waits for them before the block loads are issued)
  const int n = lane & 15, r = lane >> 4;
  const uint32_t keep = n < cols ? 0xFFFFFFFFu : 0u;
  const uint16_t* src = x.iq + (col0 + min(n, cols - 1)) * kDim;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 v = *reinterpret_cast<const uint4*>(src + 16 * r + 64 * (c >> 1) + 8 * (c & 1));
    v.x &= keep;
    v.y &= keep;
    v.z &= keep;
    v.w &= keep;
    q.b[c] = __builtin_bit_cast(bf16x8, v);
  }
  q.unscale = 1.0f;
}

// NVFP4 queries in two steps, so that the block loads can be issued between
// them: fetch() issues the raw bf16 loads (from a clamped column, masked to
// zero past cols without a branch), make() converts.
struct QueryRawNvfp4 {
  uint4 raw[4];
  __device__ __forceinline__ void fetch(const IndexArgs& x, size_t col0, int cols, int lane) {
    const int n = lane & 15, r = lane >> 4;
    const uint4* src =
        reinterpret_cast<const uint4*>(x.iq + (col0 + min(n, cols - 1)) * kDim + 32 * r);
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = src[c];
  }
  __device__ __forceinline__ void make(int cols, int lane, QueryB<kNVFP4>& q) const {
    const uint32_t keep = (lane & 15) < cols ? 0xFFFFFFFFu : 0u;
    uint32_t w[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[c][0] = raw[c].x & keep;
      w[c][1] = raw[c].y & keep;
      w[c][2] = raw[c].z & keep;
      w[c][3] = raw[c].w & keep;
    }
    // largest bf16 exponent field of column n (its 128 dims sit in lanes n,
    // n + 16, n + 32, n + 48)
    uint32_t e = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int k = 0; k < 4; ++k) e = max(e, max(w[c][k] & 0x7F80u, (w[c][k] >> 16) & 0x7F80u));
    }
    e = max(e, (uint32_t)lane_xor<16>((int)e));
    e = max(e, (uint32_t)lane_xor<32>((int)e));
    const int emax = (int)(e >> 7);        // biased exponent (0: the column is zero)
    const int sh = emax ? 142 - emax : 0;  // 2^(emax - 127 + sh) = 2^15
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = ldexpf(__uint_as_float(w[c][k] << 16), sh);
        const float hi = ldexpf(__uint_as_float(w[c][k] & 0xFFFF0000u), sh);
        o[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
      }
      q.b[c] = __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
    }
    q.unscale = ldexpf(1.0f, -sh);
  }
};

// FP8 queries: nothing to convert (fetch loads them).
struct QueryRawFp8 {
  QueryB<kFP8> q;
  __device__ __forceinline__ void fetch(const IndexArgs& x, size_t col0, int cols, int lane) {
    load_query_b(x, col0, cols, lane, q);
  }
  __device__ __forceinline__ void make(int, int, QueryB<kFP8>& out) const { out = q; }
};

// Per-lane running maxima of one block (tokens 4r + i of every tile).
struct TileMax {
  f32x4 m;
  __device__ __forceinline__ void init() { m = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY}; }
};

__device__ __forceinline__ void fold_tile(TileMax& tm, f32x4 acc, int tok, int pos) {
#pragma unroll
  for (int i = 0; i < 4; ++i) tm.m[i] = tok + i <= pos ? fmaxf(tm.m[i], acc[i]) : tm.m[i];
}

// Half a block's raw index keys, per format: issue() starts the contiguous
// loads of half h2 (tokens 64h2 .. 64h2+63) of physical block pb, streaming
// (each byte is read once); pool() stages them through the wave's LDS area
// and folds the half of logical block j (keys t <= pos) into tm.
template <int IK>
struct HalfRaw;

template <>
struct HalfRaw<kFP8> {
  uint4 r[8];  // r[i]: token 8i + lane/8 of the half, 16-byte chunk lane%8
  // STREAM: the bytes are read once (streaming hint); otherwise other waves
  // of the shared scan read them again soon, from L2.
  template <bool STREAM = true>
  __device__ __forceinline__ void issue(const IndexArgs& x, int pb, int h2, int lane) {
    const uint4* src =
        reinterpret_cast<const uint4*>(x.ikd + (size_t)pb * (kBlock * kDim)) + h2 * 512 + lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = STREAM ? load_stream(src + i * 64) : src[i * 64];
  }
  __device__ __forceinline__ void pool(int j, int h2, int pos, int lane, const QueryB<kFP8>& q,
                                       TileMax& tm, uint4* stage) const {
    // The syncs order the lanes' LDS accesses: reads of the previous half,
    // these writes, then reads of other lanes' writes.
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 8; ++i) stage[stage_slot(i, lane)] = r[i];
    wave_lds_sync();
    fold_staged(j, h2, pos, lane, q, tm, stage);
  }
  // LDS slot of the half's 16-byte chunk lane % 8 of token 8i + lane / 8:
  // token t's row is at 8t chunks, chunk c at slot c ^ (t % 8)
  __device__ static __forceinline__ int stage_slot(int i, int lane) {
    return (8 * i + (lane >> 3)) * 8 + ((lane & 7) ^ (lane >> 3));
  }
  // Folds half h2 of logical block j, staged at st, into tm (keys t <= pos).
  __device__ static __forceinline__ void fold_staged(int j, int h2, int pos, int lane,
                                                     const QueryB<kFP8>& q, TileMax& tm,
                                                     const uint4* st) {
    const int n = lane & 15, rg = lane >> 4;
    const int tok = j * kBlock + 64 * h2 + 4 * rg;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 v0 = st[(16 * t + n) * 8 + (rg ^ (n & 7))];
      const uint4 v1 = st[(16 * t + n) * 8 + ((rg + 4) ^ (n & 7))];
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = mfma_bf16(fp8x8_bf16(v0.x, v0.y), q.b[0], acc);
      acc = mfma_bf16(fp8x8_bf16(v0.z, v0.w), q.b[1], acc);
      acc = mfma_bf16(fp8x8_bf16(v1.x, v1.y), q.b[2], acc);
      acc = mfma_bf16(fp8x8_bf16(v1.z, v1.w), q.b[3], acc);
      fold_tile(tm, acc, tok + 16 * t, pos);
    }
  }
};

// NVFP4 keys: the whole block's loads are issued together -- 8 KB of E2M1
// data as eight 1 KB loads and the block's 1 KB of scales as one -- and the
// scales are staged in LDS next to the data (each lane needs the scales of
// other lanes' tokens).
struct BlockRawNvfp4 {
  uint4 d[8];  // d[i]: token 16i + lane/4 of the block, 16-byte chunk lane%4
  uint4 sc;    // the 8 scale bytes of tokens 2 lane and 2 lane + 1
  template <bool STREAM = true>
  __device__ __forceinline__ void issue(const IndexArgs& x, int pb, int lane) {
    const uint4* src = reinterpret_cast<const uint4*>(x.ikd + (size_t)pb * (kBlock * kDim / 2)) + lane;
    const uint4* ssrc =
        reinterpret_cast<const uint4*>(x.iks + (size_t)pb * (kBlock * kDim / 16)) + lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = STREAM ? load_stream(src + i * 64) : src[i * 64];
    sc = STREAM ? load_stream(ssrc) : *ssrc;
  }
  // E2M1 value x e4m3 block scale is exact in f16 (at most 6 significant
  // bits, inside [2^-10, 2688]); the tensor scale is folded into out_scale.
  // stage: 4 KB of data (half a block at a time) then the block's 1 KB of
  // scales.
  __device__ __forceinline__ void pool(int j, int pos, int lane, const QueryB<kNVFP4>& q,
                                       TileMax& tm, uint4* stage) const {
    const int n = lane & 15, rg = lane >> 4;
    const uint16_t* scl = reinterpret_cast<const uint16_t*>(stage + 256);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      // token t (0..63) of the half: row at 4t chunks, chunk p at slot p ^ ((t / 2) % 4)
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * i + (lane >> 2);
        stage[t * 4 + ((lane & 3) ^ ((t >> 1) & 3))] = d[4 * h2 + i];
      }
      if (h2 == 0) stage[256 + lane] = sc;
      wave_lds_sync();
      const int tok = j * kBlock + 64 * h2 + 4 * rg;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tt = 16 * t + n;
        const uint4 v = stage[tt * 4 + (rg ^ ((tt >> 1) & 3))];
        // scales of dims [32rg, +16) and [32rg + 16, +16) of token 64 h2 + tt
        const uint32_t s2 = scl[4 * (64 * h2 + tt) + rg];
        const f16x2 sc2 = fp8x2_to_f16x2<false>(s2);
        const f16x2 s0 = {sc2[0], sc2[0]}, s1 = {sc2[1], sc2[1]};
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = mfma_f16(nvfp4x8_f16s(v.x, s0), q.b[0], acc);
        acc = mfma_f16(nvfp4x8_f16s(v.y, s0), q.b[1], acc);
        acc = mfma_f16(nvfp4x8_f16s(v.z, s1), q.b[2], acc);
        acc = mfma_f16(nvfp4x8_f16s(v.w, s1), q.b[3], acc);
        fold_tile(tm, acc, tok + 16 * t, pos);
      }
    }
  }
};

// FP8 keys: the block as two halves (the FP8 kernel takes one block per
// wave, so nothing more needs to be in flight).
struct BlockRawFp8 {
  HalfRaw<kFP8> h[2];
  template <bool STREAM = true>
  __device__ __forceinline__ void issue(const IndexArgs& x, int pb, int lane) {
    h[0].template issue<STREAM>(x, pb, 0, lane);
    h[1].template issue<STREAM>(x, pb, 1, lane);
  }
  __device__ __forceinline__ void pool(int j, int pos, int lane, const QueryB<kFP8>& q,
                                       TileMax& tm, uint4* stage) const {
    h[0].pool(j, 0, pos, lane, q, tm, stage);
    h[1].pool(j, 1, pos, lane, q, tm, stage);
  }
};

template <int IK>
struct BlockRawOf {
  typedef BlockRawFp8 type;
  typedef QueryRawFp8 query;
};
template <>
struct BlockRawOf<kNVFP4> {
  typedef BlockRawNvfp4 type;
  typedef QueryRawNvfp4 query;
};

// The block's pooled score of group lane%16, times out_scale (lanes 0..G-1
// hold groups 0..G-1).
__device__ __forceinline__ float finish_block(const IndexArgs& x, const TileMax& tm,
                                             float unscale) {
  float m = fmaxf(fmaxf(tm.m[0], tm.m[1]), fmaxf(tm.m[2], tm.m[3]));
  m = fmaxf(m, lane_xor_f<16>(m));
  m = fmaxf(m, lane_xor_f<32>(m));
  return (m * unscale) * x.out_scale;
}

// Blocks a wave of the decode scan takes in one run (the next block's loads
// in flight while one is scored): one for FP8 keys (16 KB per block), four
// for NVFP4 keys (9 KB per block, more conversion work per byte).
template <int IK>
constexpr int blocks_per_wave() {
  return IK == kFP8 ? 1 : 4;
}

// One wave of the decode scan: row group rg (rows rg * rows_per_wave ..) of
// sequence b, blocks j0 + 4 i (i < blocks_per_wave); scores to x.scores
// ([rows][G][MB]).
template <int IK>
__device__ __forceinline__ void scan_wave_blocks(const IndexArgs& x, int b, int rg, int j0,
                                                 uint4* stage) {
  constexpr int NB = blocks_per_wave<IK>();
  const int lane = threadIdx.x & 63;
  const int r0 = rg * x.rows_per_wave, nr = min(x.rows_per_wave, x.R - r0);
  const int cols = nr * x.G;
  const size_t col0 = ((size_t)b * x.R + r0) * x.G;  // first (row, group) pair
  if (j0 >= x.MB) return;
  auto put = [&](int j, float v) {
    if (lane < cols) x.scores[(col0 + lane) * x.MB + j] = v;
  };
  // table entries of the wave's blocks, lane i holding block i's (issued
  // alongside the length loads)
  int entry = -1;
  if (lane < NB && j0 + 4 * lane < x.MB) entry = x.bt[(size_t)b * x.MB + j0 + 4 * lane];
  // this lane's column: its row's last visible key (-1 past the columns)
  const int n = lane & 15;
  const int pos = n < cols ? row_last_key(x.lens, x.qpos, b * x.R + r0 + n / x.G, b, x.MB) : -1;
  int pos_max = pos;  // the wave's furthest-seeing column
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) pos_max = max(pos_max, __shfl_xor(pos_max, o, 64));
  // the wave's blocks with keys to see: a prefix of its run (blocks past
  // every column's last key, or past the table, score -inf unread)
  int live = 0;
#pragma unroll
  for (int i = 0; i < NB; ++i)
    live += (j0 + 4 * i < x.MB && (j0 + 4 * i) * kBlock <= pos_max) ? 1 : 0;
  for (int i = live; i < NB && j0 + 4 * i < x.MB; ++i) put(j0 + 4 * i, -INFINITY);
  if (live == 0) return;
  // physical block of the wave's i-th block, -1 for an entry outside the pool
  auto phys = [&](int i) {
    const int e = __builtin_amdgcn_readlane(entry, i);
    return (e < 0 || e >= x.P) ? -1 : e;
  };
  // Every load of the loop is issued unconditionally (a branch around an
  // issue makes the compiler wait for all loads in flight where the paths
  // join, which would serialise the blocks): loads for an unusable block
  // read physical block 0 (in range; the result is not used).
  typename BlockRawOf<IK>::query qraw;
  qraw.fetch(x, col0, cols, lane);
  typename BlockRawOf<IK>::type buf[2];
  int pb = phys(0);
  buf[0].issue(x, max(pb, 0), lane);
  QueryB<IK> q;
  qraw.make(cols, lane, q);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (i >= live) break;
    const int j = j0 + 4 * i;
    const int pb_next = i + 1 < live ? phys(i + 1) : -1;
    if (i + 1 < NB) buf[(i + 1) & 1].issue(x, max(pb_next, 0), lane);
    if (pb < 0) {  // an entry outside the pool: the block contributes nothing
      put(j, -INFINITY);
    } else {
      TileMax tm;
      tm.init();
      buf[i & 1].pool(j, pos, lane, q, tm, stage);
      put(j, finish_block(x, tm, q.unscale));
    }
    pb = pb_next;
  }
}

}  // namespace msa
