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
  float out_scale;    // index_scale * index_k_scale (NVFP4: times the tensor scale)
};

// Lanes 0..cols-1 store block j's scores of the wave's columns: column c is
// (row, group) pair col0 + c of the [rows][G] order.
__device__ __forceinline__ void put_block_scores(const IndexArgs& x, size_t col0, int cols, int j,
                                                 int lane, float v) {
  if (lane < cols) x.scores[(col0 + lane) * x.MB + j] = v;
}

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

constexpr int kStageBytes = 8192;  // LDS per wave: half a block (FP8) staged

// B operand: the wave's cols index queries, (row, group) pairs col0 ..
// col0 + cols - 1 (zero columns past cols).
struct QueryB {
  bf16x8 b[4];
};

template <int IK>
__device__ __forceinline__ void load_query_b(const IndexArgs& x, size_t col0, int cols, int lane,
                                             QueryB& q) {
  const int n = lane & 15, r = lane >> 4;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int d = IK == kFP8 ? 16 * r + 64 * (c >> 1) + 8 * (c & 1) : 32 * r + 8 * c;
    q.b[c] = n < cols ? *reinterpret_cast<const bf16x8*>(x.iq + (col0 + n) * kDim + d)
                      : bf16x8{};
  }
}

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
  __device__ __forceinline__ void issue(const IndexArgs& x, int pb, int h2, int lane) {
    const uint4* src =
        reinterpret_cast<const uint4*>(x.ikd + (size_t)pb * (kBlock * kDim)) + h2 * 512 + lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = load_stream(src + i * 64);
  }
  __device__ __forceinline__ void pool(int j, int h2, int pos, int lane, const QueryB& q,
                                       TileMax& tm, uint4* stage) const {
    // token t (0..63) row at 8t chunks; chunk c at slot c ^ (t % 8).  The
    // syncs order the lanes' LDS accesses: reads of the previous half, these
    // writes, then reads of other lanes' writes.
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 8; ++i) stage[(8 * i + (lane >> 3)) * 8 + ((lane & 7) ^ (lane >> 3))] = r[i];
    wave_lds_sync();
    const int n = lane & 15, rg = lane >> 4;
    const int tok = j * kBlock + 64 * h2 + 4 * rg;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 v0 = stage[(16 * t + n) * 8 + (rg ^ (n & 7))];
      const uint4 v1 = stage[(16 * t + n) * 8 + ((rg + 4) ^ (n & 7))];
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = mfma_bf16(fp8x8_bf16(v0.x, v0.y), q.b[0], acc);
      acc = mfma_bf16(fp8x8_bf16(v0.z, v0.w), q.b[1], acc);
      acc = mfma_bf16(fp8x8_bf16(v1.x, v1.y), q.b[2], acc);
      acc = mfma_bf16(fp8x8_bf16(v1.z, v1.w), q.b[3], acc);
      fold_tile(tm, acc, tok + 16 * t, pos);
    }
  }
};

template <>
struct HalfRaw<kNVFP4> {
  uint4 d[4];     // d[i]: token 16i + lane/4 of the half, 16-byte chunk lane%4
  uint32_t s[4];  // s[t]: the two e4m3 scales of token 16t + lane%16, dims [32r, +32)
  __device__ __forceinline__ void issue(const IndexArgs& x, int pb, int h2, int lane) {
    const uint4* src =
        reinterpret_cast<const uint4*>(x.ikd + (size_t)pb * (kBlock * kDim / 2)) + h2 * 256 + lane;
    const uint16_t* ss = reinterpret_cast<const uint16_t*>(
                             x.iks + (size_t)pb * (kBlock * kDim / 16) +
                             (size_t)(64 * h2 + (lane & 15)) * (kDim / 16)) + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[i] = load_stream(src + i * 64);
      s[i] = __builtin_nontemporal_load(ss + i * 64);
    }
  }
  // E2M1 value x e4m3 block scale is exact in bf16 (at most 6 significant
  // bits, inside bf16's range); the tensor scale is folded into out_scale.
  __device__ __forceinline__ void pool(int j, int h2, int pos, int lane, const QueryB& q,
                                       TileMax& tm, uint4* stage) const {
    // token t (0..63) row at 4t chunks; chunk p at slot p ^ ((t / 2) % 4)
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * i + (lane >> 2);
      stage[t * 4 + ((lane & 3) ^ ((t >> 1) & 3))] = d[i];
    }
    wave_lds_sync();
    const int n = lane & 15, rg = lane >> 4;
    const int tok = j * kBlock + 64 * h2 + 4 * rg;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tt = 16 * t + n;
      const uint4 v = stage[tt * 4 + (rg ^ ((tt >> 1) & 3))];
      const f32x2 sc = fp8x2_to_f32x2<false>(s[t]);  // dims [32r, +16), [32r+16, +16)
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = mfma_bf16(nvfp4x8_bf16(v.x, sc[0]), q.b[0], acc);
      acc = mfma_bf16(nvfp4x8_bf16(v.y, sc[0]), q.b[1], acc);
      acc = mfma_bf16(nvfp4x8_bf16(v.z, sc[1]), q.b[2], acc);
      acc = mfma_bf16(nvfp4x8_bf16(v.w, sc[1]), q.b[3], acc);
      fold_tile(tm, acc, tok + 16 * t, pos);
    }
  }
};

// The block's pooled score of group lane%16, times out_scale (lanes 0..G-1
// hold groups 0..G-1).
__device__ __forceinline__ float finish_block(const IndexArgs& x, const TileMax& tm) {
  float m = fmaxf(fmaxf(tm.m[0], tm.m[1]), fmaxf(tm.m[2], tm.m[3]));
  m = fmaxf(m, lane_xor_f<16>(m));
  m = fmaxf(m, lane_xor_f<32>(m));
  return m * x.out_scale;
}

}  // namespace msa
