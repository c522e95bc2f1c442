// prefill_index.hip -- indexer scores + block max-pool for many query rows
// per sequence (chunked prefill, speculative decode) as a dense MFMA
// contraction.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer", and its list of MSA kernels, which names an indexer prefill
// kernel): every query row r of a sequence scores the keys it can see (t <=
// pos_r) with one index query per group, and the scores are max-pooled per
// 128-token block.  With many rows per sequence this is the dense product
// Q [rows*G x 128] . K^T [128 x tokens] with a causal mask, followed by a
// per-block max: MFMA-bound, not HBM-bound, because every key serves every
// row of its sequence.
//
// Work decomposition: a workgroup takes a tile of 256 consecutive (row,
// group) columns of one sequence (wave w: columns 64w .. 64w+63 as four
// 16-column MFMA tiles, held as B operands for the whole kernel) and a range
// of 16 logical blocks (small ranges make many workgroups, so the partial
// last wave of them is a small share of the run).  Per block, the 256 threads
// move its 16 KB of e4m3 keys from HBM straight into LDS with LDS-direct
// loads (the next block's while the current one computes), each lane fetching
// the 16-byte chunk that belongs at its LDS slot, so the chunks land swizzled
// (chunk c of token t at slot c ^ (t % 8), free of bank conflicts); each wave
// then runs S^T = K Q^T on v_mfma_f32_16x16x32_bf16 for its 64 columns over
// the block's 8 tiles of 16 tokens, keeping a masked running max per column.
// The per-block maxima gather in LDS and leave as 64-byte runs per column.
//
// NVFP4 index keys (API reference of MiniMaxM3SparseAttention: FP4 index
// cache; blog section "AMD NVFP4 MSA kernels") stage 9 KB per block: 8 KB of
// E2M1 data (token rows of 64 bytes, chunk c of token t at slot
// c ^ ((t / 4) % 4)) and the block's 1 KB of e4m3 scales (one per 16 dims).
//
// Arithmetic: e4m3 keys convert exactly to bf16; products with the bf16
// index queries are exact and accumulate in fp32.  An E2M1 value times its
// e4m3 scale is exact in f16 (at most 6 significant bits, inside [2^-10,
// 2688]), so NVFP4 keys run on v_mfma_f32_16x16x32_f16 against f16 queries,
// each column shifted by a power of two that puts its largest element in
// [2^15, 2^16) (every element within 2^32 of it converts exactly); the shift
// is undone on the pooled maximum, which commutes with a positive power-of-
// two scale.  Blocks past a row's last visible key, and table entries
// outside the pool, give -inf.
#include "device.hpp"
#include "launch.hpp"

namespace msa {

constexpr int kCols = 256;   // (row, group) columns per workgroup
constexpr int kRange = 16;   // logical blocks per workgroup

// 16 bytes per lane from global memory straight into LDS (no registers):
// lane i's bytes land at wave_base + 16 i, so wave_base must be the same
// for the whole wave.
__device__ __forceinline__ void load_lds16(const uint4* src, uint4* wave_base) {
  __builtin_amdgcn_global_load_lds(
      (__attribute__((address_space(1))) void*)(const_cast<uint4*>(src)),
      (__attribute__((address_space(3))) void*)wave_base, 16, 0, 0);
}
// wait until every vector-memory operation of this thread has completed,
// LDS-direct loads included
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

struct PrefillArgs {
  const uint16_t* iq;  // [rows][G][128] bf16
  const uint8_t* ik;   // [P][128][128] e4m3, or NVFP4 data [P][128][64]
  const uint8_t* iks;  // NVFP4: [P][128][8] e4m3 scales
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* qpos;
  float* scores;  // [rows][G][MB]
  int R, G, MB, P;
  int tiles_per_seq;  // ceil(R*G / kCols)
  float out_scale;
};

// Staged block bytes (16-byte chunks) and the B operand type of each key format.
template <int IK>
constexpr int stage_chunks() {
  return IK == kFP8 ? kBlock * kDim / 16 : kBlock * kDim / 32 + kBlock * kDim / 256;
}
template <int IK>
struct PrefillB {
  typedef bf16x8 type;
};
template <>
struct PrefillB<kNVFP4> {
  typedef f16x8 type;
};

// A operand chunk k (k = 0..3) of token tok for lane group r, from the
// staged block.  FP8: dims 16r + 64(k/2) + 8(k%2) + 0..7 as bf16.  NVFP4: dims
// 32r + 8k + 0..7 as f16 (E2M1 x its e4m3 scale).
template <int IK>
struct KeyChunks;
template <>
struct KeyChunks<kFP8> {
  bf16x8 a[4];
  __device__ __forceinline__ KeyChunks(const uint4* __restrict__ stage, int tok, int r) {
    const uint4 v0 = stage[tok * 8 + (r ^ (tok & 7))];
    const uint4 v1 = stage[tok * 8 + ((r + 4) ^ (tok & 7))];
    a[0] = fp8x8_bf16(v0.x, v0.y);
    a[1] = fp8x8_bf16(v0.z, v0.w);
    a[2] = fp8x8_bf16(v1.x, v1.y);
    a[3] = fp8x8_bf16(v1.z, v1.w);
  }
};
template <>
struct KeyChunks<kNVFP4> {
  f16x8 a[4];
  __device__ __forceinline__ KeyChunks(const uint4* __restrict__ stage, int tok, int r) {
    const uint4 v = stage[tok * 4 + (r ^ ((tok >> 2) & 3))];
    // scales 2r (dims 32r .. +15) and 2r + 1 (dims 32r + 16 .. +31) of the token
    const uint32_t s2 = reinterpret_cast<const uint16_t*>(stage + kBlock * kDim / 32)[tok * 4 + r];
    const f16x2 sc = fp8x2_to_f16x2<false>(s2);
    const f16x2 s0 = {sc[0], sc[0]}, s1 = {sc[1], sc[1]};
    a[0] = nvfp4x8_f16s(v.x, s0);
    a[1] = nvfp4x8_f16s(v.y, s0);
    a[2] = nvfp4x8_f16s(v.z, s1);
    a[3] = nvfp4x8_f16s(v.w, s1);
  }
};

__device__ __forceinline__ f32x4 mfma_k(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return mfma_bf16(a, b, c);
}
__device__ __forceinline__ f32x4 mfma_k(const f16x8& a, const f16x8& b, const f32x4& c) {
  return mfma_f16(a, b, c);
}

// S^T for two 16-token tiles of the staged block against the wave's four
// 16-column tiles, folded into the running maxima m (D row 4r + i of a tile
// is key 16u + 4r + i, column 16t + n).  The four accumulators of a tile are
// independent chains, issued interleaved so that no MFMA waits on the one
// before it; the maxima take both tiles in one three-input max.  MASKED:
// keys past a column's last visible key count as -inf.
template <int IK, bool FULL>
__device__ __forceinline__ void block_max(const uint4* __restrict__ stage,
                                          const typename PrefillB<IK>::type (&qb)[4][4],
                                          const int (&cpos)[4], int j, int n, int r,
                                          f32x4 (&m)[4]) {
#pragma unroll 1
  for (int u = 0; u < 8; u += 2) {
    f32x4 acc[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const KeyChunks<IK> kc(stage, 16 * (u + h) + n, r);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[h][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[h][t] = mfma_k(kc.a[k], qb[t][k], acc[h][t]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x0 = acc[0][t][i], x1 = acc[1][t][i];
        if constexpr (!FULL) {
          const int key = j * kBlock + 16 * u + 4 * r + i;
          x0 = key <= cpos[t] ? x0 : -INFINITY;
          x1 = key + 16 <= cpos[t] ? x1 : -INFINITY;
        }
        m[t][i] = __builtin_fmaxf(m[t][i], __builtin_fmaxf(x0, x1));
      }
    }
  }
}

// B operands of one column: FP8 keys take the bf16 queries as they are
// (unscale 1); NVFP4 keys take them as f16, shifted by 2^sh so that the
// column's largest element lands in [2^15, 2^16), with unscale = 2^-sh.  The
// column's 128 dims sit in lanes n, n + 16, n + 32, n + 48 (lane group r);
// `raw` holds the lane's four 16-byte chunks in the format's dim order.
__device__ __forceinline__ void make_b(const uint4 (&raw)[4], bf16x8 (&b)[4], float& unscale) {
#pragma unroll
  for (int k = 0; k < 4; ++k) b[k] = __builtin_bit_cast(bf16x8, raw[k]);
  unscale = 1.0f;
}
__device__ __forceinline__ void make_b(const uint4 (&raw)[4], f16x8 (&b)[4], float& unscale) {
  uint32_t e = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) e = max(e, max(w[q] & 0x7F80u, (w[q] >> 16) & 0x7F80u));
  }
  e = max(e, (uint32_t)lane_xor<16>((int)e));
  e = max(e, (uint32_t)lane_xor<32>((int)e));
  const int emax = (int)(e >> 7);        // biased exponent (0: the column is zero)
  const int sh = emax ? 142 - emax : 0;  // 2^(emax - 127 + sh) = 2^15
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = ldexpf(__uint_as_float(w[q] << 16), sh);
      const float hi = ldexpf(__uint_as_float(w[q] & 0xFFFF0000u), sh);
      o[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    b[k] = __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
  }
  unscale = ldexpf(1.0f, -sh);
}

template <int IK>
__global__ __launch_bounds__(256, 3) void prefill_index_kernel(PrefillArgs x) {
  // two staged key blocks, swizzled; two arrays rather than one [2][...] so
  // that the compiler sees the reads of one and the LDS-direct loads into the
  // other as disjoint and does not wait for those loads before the reads
  constexpr int SC = stage_chunks<IK>();
  __shared__ uint4 stage0[SC];
  __shared__ uint4 stage1[SC];
  __shared__ float smax[kCols][kRange + 1];       // per-column block maxima (+1: no bank conflicts)
  __shared__ int s_pos_max;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int b = blockIdx.x / x.tiles_per_seq, tile = blockIdx.x % x.tiles_per_seq;
  const int seq_cols = x.R * x.G;
  const int col0 = tile * kCols;  // first column of the tile within the sequence
  const int ncols = min(kCols, seq_cols - col0);
  const int j0 = blockIdx.y * kRange, j1 = min(x.MB, j0 + kRange);
  const int n = lane & 15, r = lane >> 4;

  // ---- B operands and visibility of this lane's four columns ----
  typename PrefillB<IK>::type qb[4][4];
  float unscale[4];
  int cpos[4];
  int pos_lo = 0x7FFFFFFF, pos_hi = -1;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = 64 * wave + 16 * t + n;  // column within the tile
    const bool valid = c < ncols;
    const int flat = b * seq_cols + col0 + c;  // (row, group) index
    const int row = flat / x.G;
    cpos[t] = valid ? row_last_key(x.lens, x.qpos, row, b, x.MB) : -1;
    uint4 raw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = IK == kFP8 ? 16 * r + 64 * (k >> 1) + 8 * (k & 1) : 32 * r + 8 * k;
      raw[k] = valid ? *reinterpret_cast<const uint4*>(x.iq + (size_t)flat * kDim + d)
                     : make_uint4(0, 0, 0, 0);
    }
    make_b(raw, qb[t], unscale[t]);
    if (valid) {
      pos_lo = min(pos_lo, cpos[t]);
      pos_hi = max(pos_hi, cpos[t]);
    }
  }
  // wave-uniform bounds: every column of the wave sees keys <= wave_lo; none
  // sees keys > wave_hi
  int wave_lo = pos_lo, wave_hi = pos_hi;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    wave_lo = min(wave_lo, __shfl_xor(wave_lo, o, 64));
    wave_hi = max(wave_hi, __shfl_xor(wave_hi, o, 64));
  }
  if (threadIdx.x == 0) s_pos_max = -1;
  for (int i = threadIdx.x; i < kCols * (kRange + 1); i += 256) (&smax[0][0])[i] = -INFINITY;
  __syncthreads();
  if (lane == 0) atomicMax(&s_pos_max, wave_hi);
  __syncthreads();
  // blocks this workgroup computes: [j0, jend)
  const int jend = min(j1, s_pos_max < 0 ? j0 : s_pos_max / kBlock + 1);

  // ---- stream the blocks: HBM -> LDS (swizzled, no registers) -> MFMA ----
  const int32_t* brow = x.bt + (size_t)b * x.MB;
  int next_e = 0;  // table entry of the block being loaded
  auto issue = [&](int j, uint4* stg) {
    const int e = brow[j];
    next_e = e;
    const int pb = e >= 0 && e < x.P ? e : 0;  // invalid entries are masked below
    if constexpr (IK == kFP8) {
      const uint4* src = reinterpret_cast<const uint4*>(x.ik + (size_t)pb * (kBlock * kDim));
      // slot s = 256 i + thread of the stage holds chunk (s % 8) ^ (tok % 8)
      // of token tok = s / 8; the wave's 64 slots of instruction i are
      // contiguous
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 256 * i + (int)threadIdx.x;
        const int tok = slot >> 3, c = (slot & 7) ^ (tok & 7);
        load_lds16(src + tok * 8 + c, stg + 256 * i + 64 * wave);
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(x.ik + (size_t)pb * (kBlock * kDim / 2));
      // data: slot s = 256 i + thread holds chunk (s % 4) ^ ((tok / 4) % 4)
      // of token tok = s / 4
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int slot = 256 * i + (int)threadIdx.x;
        const int tok = slot >> 2, c = (slot & 3) ^ ((tok >> 2) & 3);
        load_lds16(src + tok * 4 + c, stg + 256 * i + 64 * wave);
      }
      // scales: the block's 1 KB, in order, by the first wave
      if (wave == 0) {
        const uint4* ssrc =
            reinterpret_cast<const uint4*>(x.iks + (size_t)pb * (kBlock * kDim / 16));
        load_lds16(ssrc + lane, stg + kBlock * kDim / 32);
      }
    }
  };
  // block j from stage `cur`, while block j + 1 loads into `nxt`
  auto step = [&](int j, const uint4* cur, uint4* nxt) {
    const int e = next_e;  // block j's table entry
    wait_vm_all();         // this thread's part of block j is in LDS
    __syncthreads();       // every part is; the other stage's readers are done
    if (j + 1 < jend) issue(j + 1, nxt);
    if (e < 0 || e >= x.P) return;     // invalid table entry: the block stays -inf
    if (j * kBlock > wave_hi) return;  // no column of this wave sees the block
    // wave-uniform: every column of the wave sees the whole block
    const bool full = __builtin_amdgcn_readfirstlane((int)(j * kBlock + kBlock - 1 <= wave_lo));
    f32x4 m[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) m[t] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (full)
      block_max<IK, true>(cur, qb, cpos, j, n, r, m);
    else
      block_max<IK, false>(cur, qb, cpos, j, n, r, m);
    // max over the lane's 4 keys and the 4 lane groups: lanes 0..15 keep
    // column 16t + n's block maximum
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float v = fmaxf(fmaxf(m[t][0], m[t][1]), fmaxf(m[t][2], m[t][3]));
      v = fmaxf(v, lane_xor_f<16>(v));
      v = fmaxf(v, lane_xor_f<32>(v));
      if (r == 0) smax[64 * wave + 16 * t + n][j - j0] = v * unscale[t] * x.out_scale;
    }
  };
  if (j0 < jend) issue(j0, stage0);
  for (int j = j0; j < jend; j += 2) {  // jend is the same for the whole workgroup
    step(j, stage0, stage1);
    if (j + 1 < jend) step(j + 1, stage1, stage0);
  }
  __syncthreads();
  // ---- column c's blocks [j0, j1): one contiguous run each ----
  const int c = threadIdx.x;
  if (c < ncols) {
    float* dst = x.scores + (size_t)(b * seq_cols + col0 + c) * x.MB + j0;
    for (int k = 0; k < j1 - j0; ++k) dst[k] = smax[c][k];
  }
}

bool prefill_index_supported(const Shape& s) {
  return (s.ik_dtype == kFP8 || s.ik_dtype == kNVFP4) && s.R >= 16;
}

hipError_t launch_prefill_index_scores(const Shape& s, const void* index_q, const void* ik_data,
                                       const void* ik_scales, const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* q_pos, float* scores, hipStream_t st) {
  PrefillArgs x;
  x.iq = static_cast<const uint16_t*>(index_q);
  x.ik = static_cast<const uint8_t*>(ik_data);
  x.iks = static_cast<const uint8_t*>(ik_scales);
  x.bt = block_table;
  x.lens = seq_lens;
  x.qpos = q_pos;
  x.scores = scores;
  x.R = s.R;
  x.G = s.G;
  x.MB = s.MB;
  x.P = s.P;
  x.tiles_per_seq = (s.R * s.G + kCols - 1) / kCols;
  x.out_scale = s.index_scale * s.ik_scale;
  const int nseq = s.rows / s.R;
  const dim3 grid((unsigned)(nseq * x.tiles_per_seq), (unsigned)((s.MB + kRange - 1) / kRange));
  if (grid.x == 0) return hipSuccess;
  if (s.ik_dtype == kFP8)
    hipLaunchKernelGGL(prefill_index_kernel<kFP8>, grid, dim3(256), 0, st, x);
  else
    hipLaunchKernelGGL(prefill_index_kernel<kNVFP4>, grid, dim3(256), 0, st, x);
  return hipGetLastError();
}

}  // namespace msa
