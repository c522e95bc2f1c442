// index_scores.hip -- lightning-indexer scoring + per-block max-pool.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer"): every cached key is scored by one index query per GQA group
// against one shared index-key head; the scores are max-pooled to one score
// per 128-token block.  Decode is HBM-bound: the scan reads 128 B per token
// (FP8) or 72 B (NVFP4), so these kernels stream each block once, coalesced,
// and keep all arithmetic in registers.
//
// Work decomposition: one wavefront per (logical block, group of up to 16 / G
// rows of one sequence); four wavefronts per workgroup take four consecutive
// blocks.
// Every load instruction of a wave reads 1 KB of consecutive bytes, and a
// block's loads are all issued before any arithmetic, to keep many bytes in
// flight per wave.  Blocks past a row's last visible key, and block-table
// entries outside the pool, produce -inf without touching the cache.
//
// Arithmetic: keys are converted exactly to bf16 (e4m3 and e2m1 values are
// bf16-representable) and multiplied with the bf16 index queries on MFMA
// (index_block.hpp): exact products, fp32 accumulation.  The fp32 path uses
// plain fp32 FMAs.  The positive score scale commutes with the max, so it is
// applied once per block.
#include "device.hpp"
#include "index_block.hpp"
#include "launch.hpp"

namespace msa {

// -------------------------------------------------------------------------
// FP8 e4m3 / NVFP4 index keys, bf16 index queries: one wave per (row group,
// run of NB blocks), on MFMA (the layouts and arithmetic are those of
// index_block.hpp).  A row group is up to 16 / G consecutive rows of one
// sequence (R > 1: speculative-decode rows, each with its own last visible
// key); its rows_per_wave * G index queries are the MFMA's columns, so the
// block's keys are read once for all of them.
// Wave w of workgroup x takes blocks 4 NB x + w + 4 i (i < NB).  The loads of
// block i + 1 are issued before block i is scored, so a wave keeps two
// blocks in flight while it computes: with NB = 1 a wave streams nothing
// while it converts and multiplies, which costs little for FP8 (16 KB per
// block, little arithmetic per byte) but starved the NVFP4 scan (9 KB per
// block, more conversion work per byte).
// -------------------------------------------------------------------------
template <int IK>
__global__ __launch_bounds__(256, 4) void index_mfma_kernel(IndexArgs x) {
  __shared__ uint4 stage[4][stage_bytes<IK>() / 16];  // one staging area per wave
  const int wave = wave_id();
  const int b = blockIdx.y / x.row_groups, rg = blockIdx.y % x.row_groups;
  scan_wave_blocks<IK>(x, b, rg, blockIdx.x * (4 * blocks_per_wave<IK>()) + wave, stage[wave]);
}

// -------------------------------------------------------------------------
// Shared scan (one row per sequence, share groups of consecutive sequences
// that may map logical blocks to the same physical blocks -- requests with a
// common prefix).  A wave takes a slice of up to share_per_wave(G) sequences
// of a group (their (sequence, group) columns fit one MFMA column tile) and
// one logical block j; the four waves of a workgroup take four consecutive
// slices of the same group and the same j, and every workgroup of block j
// has the same index mod 8, which the dispatcher places on one XCD: all
// requests for a block the group shares meet in one XCD's L2, at about the
// same time, and the block comes from HBM once (the loads keep their lines
// in L2 for that, unlike the streaming loads of index_mfma_kernel).  FP8
// keys: where all four waves start with the same physical block, the
// workgroup loads it once and stages it in LDS for all four (a quarter of
// the L2 reads of a block per wave, measured 3 % faster on 64 requests over a
// 131,072-token prefix).  A wave reads its slice's table entries for j and
// scores each distinct physical block among them once, for exactly the
// columns whose sequence maps j to it (and sees it): a shared prefix block
// is read once per slice, a private block once for its own sequence, and a
// slice holds few enough sequences that its private blocks (one load after
// another) stay short.  Each column is scored by the same arithmetic as in
// index_mfma_kernel, so the scores are those of the unshared scan, bit for
// bit.
// -------------------------------------------------------------------------
__host__ __device__ constexpr int share_per_wave(int G) { return G >= 8 ? 2 : 4; }

template <int IK>
__device__ __forceinline__ void index_shared_body(const IndexArgs& x, int wgs_per_group,
                                                  int wgs_per_block) {
  __shared__ uint4 stage[4][stage_bytes<IK>() / 16];  // one staging area per wave
  __shared__ int wave_e[4];
  const int lane = threadIdx.x & 63, wave = wave_id();
  // blockIdx.x = ((jr / 8) * wgs_per_block + r) * 8 + jr % 8 with
  // jr = MBp - 1 - j (MBp: MB rounded up to a multiple of 8): the last blocks
  // first, so that the private blocks past a common prefix -- the slices'
  // longest chains of loads -- start early rather than form the tail
  const int mbp = (x.MB + 7) / 8 * 8;
  const int jr = (blockIdx.x / (8 * wgs_per_block)) * 8 + (blockIdx.x & 7);
  const int j = mbp - 1 - jr;
  const int r = (blockIdx.x >> 3) % wgs_per_block;
  const int grp = r / wgs_per_group, sl = 4 * (r % wgs_per_group) + wave;
  const int spw = share_per_wave(x.G);
  const int b0 = grp * x.share + sl * spw;
  const int ns = min(min(spw, x.share - sl * spw), x.B - b0);  // the wave's sequences
  if (j >= x.MB) return;  // the same j for the whole workgroup
  // a wave past the group's last sequence has no columns but stays for the
  // workgroup's barriers
  const int cols = ns > 0 ? ns * x.G : 0;
  const size_t col0 = (size_t)b0 * x.G;  // first (row, group) pair (one row per sequence)
  // lane i < ns: sequence b0 + i's table entry and last visible key
  int entry = -1, spos = -1;
  if (lane < ns) {
    entry = x.bt[(size_t)(b0 + lane) * x.MB + j];
    spos = row_last_key(x.lens, x.qpos, b0 + lane, b0 + lane, x.MB);
  }
  const bool usable = lane < ns && j * kBlock <= spos && entry >= 0 && entry < x.P;
  uint64_t pending = __ballot(usable);
  // this lane's column n (sequence n / G): its sequence's last key
  const int n = lane & 15;
  const int pc = __shfl(spos, min(n, cols - 1) / x.G, 64);
  const int posc = n < cols ? pc : -1;
  TileMax tm;
  tm.init();
  float unscale = 1.0f;
  typename BlockRawOf<IK>::query qr;
  QueryB<IK> q;
  if (pending) {
    qr.fetch(x, col0, cols, lane);
    qr.make(cols, lane, q);
    unscale = q.unscale;
  }
  if constexpr (IK == kFP8) {
    // A block that every wave needing one takes first (a shared prefix
    // block): the workgroup reads it once, 4 KB per wave, and stages it in
    // the first two waves' LDS areas in the layout HalfRaw<kFP8> stages a
    // half in; each wave then folds it for its own columns, with the same
    // arithmetic as the per-wave path.
    const int e_w = pending ? __builtin_amdgcn_readlane(entry, __builtin_ctzll(pending)) : -1;
    if (lane == 0) wave_e[wave] = e_w;
    __syncthreads();
    int E = -1;
    bool common = true;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int ew = wave_e[w];
      if (ew >= 0) {
        if (E < 0) E = ew;
        common = common && ew == E;
      }
    }
    if (E >= 0 && common) {  // the same decision in every wave
      uint4* sh = &stage[0][0];
      const uint4* src = reinterpret_cast<const uint4*>(x.ikd + (size_t)E * (kBlock * kDim));
      uint4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = src[threadIdx.x + 256 * k];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int u = threadIdx.x + 256 * k;  // chunk u % 64 of token (u % 512) / 64 .. of half u / 512
        sh[(u >> 9) * 512 + HalfRaw<kFP8>::stage_slot((u & 511) >> 6, u & 63)] = v[k];
      }
      __syncthreads();
      const uint64_t same = __ballot(lane < ns && entry == E) & pending;
      pending &= ~same;
      const int pact = (n < cols && ((same >> (n / x.G)) & 1)) ? posc : -1;
      HalfRaw<kFP8>::fold_staged(j, 0, pact, lane, q, tm, sh);
      HalfRaw<kFP8>::fold_staged(j, 1, pact, lane, q, tm, sh + 512);
      __syncthreads();  // the per-wave loop below reuses these LDS areas
    }
  }
  {
    while (pending) {  // the distinct physical blocks, one at a time
      const int leader = __builtin_ctzll(pending);
      const int e = __builtin_amdgcn_readlane(entry, leader);
      const uint64_t same = __ballot(lane < ns && entry == e) & pending;
      pending &= ~same;
      // keys this lane's column folds from block e (-1: not its block)
      const int pact = (n < cols && ((same >> (n / x.G)) & 1)) ? posc : -1;
      typename BlockRawOf<IK>::type raw;
      raw.template issue<false>(x, e, lane);
      raw.pool(j, pact, lane, q, tm, stage[wave]);
    }
  }
  const float v = finish_block(x, tm, unscale);  // -inf for columns that see nothing
  if (lane < cols) x.scores[(col0 + lane) * x.MB + j] = v;
}

// FP8 keys: held to 128 registers, four waves per SIMD (it fits without
// spilling); NVFP4 keys need no bound for that.
__global__ __launch_bounds__(256, 4) void index_shared_fp8_kernel(IndexArgs x, int wgs_per_group,
                                                                  int wgs_per_block) {
  index_shared_body<kFP8>(x, wgs_per_group, wgs_per_block);
}
// Held to 5 waves per SIMD (94 VGPRs, no spills); unbounded it took 117
// VGPRs and 8 AGPRs, 4 waves per SIMD, and ran about 2 % slower.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void
index_shared_nvfp4_kernel(IndexArgs x, int wgs_per_group, int wgs_per_block) {
  index_shared_body<kNVFP4>(x, wgs_per_group, wgs_per_block);
}

// -------------------------------------------------------------------------
// fp32 index keys and queries (small exactness workloads).  One wave per
// block, two tokens per lane, fp32 FMA.
// -------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void index_f32_kernel(
    const float* __restrict__ iq, const float* __restrict__ ik,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ qpos, float* __restrict__ scores, int R, int MB, int P,
    float out_scale) {
  __shared__ float qs[G * kDim];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int row = blockIdx.y, b = row / R;
  for (int i = threadIdx.x; i < G * kDim; i += 256) qs[i] = iq[(size_t)row * G * kDim + i];
  __syncthreads();
  const int j = blockIdx.x * 4 + wave;
  if (j >= MB) return;
  const int entry = bt[(size_t)b * MB + j];  // issued alongside the length loads
  const int pos = row_last_key(lens, qpos, row, b, MB);
  float* out = scores + (size_t)row * G * MB + j;
  const int pb = j * kBlock > pos ? -1 : entry;
  if (pb < 0 || pb >= P) {  // past the row's last key (or an invalid table entry)
    if (lane < G) out[(size_t)lane * MB] = -INFINITY;
    return;
  }
  float m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = -INFINITY;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int tt = lane + 64 * half;
    const float4* krow =
        reinterpret_cast<const float4*>(ik + ((size_t)pb * kBlock + tt) * kDim);
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.0f;
#pragma unroll 4
    for (int d4 = 0; d4 < kDim / 4; ++d4) {
      const float4 k = krow[d4];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        acc[g] = fmaf(qs[g * kDim + 4 * d4], k.x, acc[g]);
        acc[g] = fmaf(qs[g * kDim + 4 * d4 + 1], k.y, acc[g]);
        acc[g] = fmaf(qs[g * kDim + 4 * d4 + 2], k.z, acc[g]);
        acc[g] = fmaf(qs[g * kDim + 4 * d4 + 3], k.w, acc[g]);
      }
    }
    const bool valid = j * kBlock + tt <= pos;
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = valid ? fmaxf(m[g], acc[g]) : m[g];
  }
  float v = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = m[g];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, shfl_xor(x, o));
    if (lane == g) v = x;
  }
  if (lane < G) out[(size_t)lane * MB] = v * out_scale;
}

template <int G>
static hipError_t launch_f32(const Shape& s, const void* iq, const void* ikd, const int32_t* bt,
                             const int32_t* lens, const int32_t* qpos, float* scores,
                             hipStream_t st) {
  dim3 grid((s.MB + 3) / 4, s.rows), block(256);
  hipLaunchKernelGGL(index_f32_kernel<G>, grid, block, 0, st, (const float*)iq,
                     (const float*)ikd, bt, lens, qpos, scores, s.R, s.MB, s.P,
                     s.index_scale * s.ik_scale);
  return hipGetLastError();
}

hipError_t launch_index_scores(const Shape& s, const void* index_q, const void* ik_data,
                               const void* ik_scales, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* q_pos,
                               float* scores, hipStream_t st) {
  if (prefill_index_supported(s)) {
    return launch_prefill_index_scores(s, index_q, ik_data, ik_scales, block_table, seq_lens,
                                       q_pos, scores, st);
  }
  if (s.ik_dtype == kF32) {
    switch (s.G) {
      case 1: return launch_f32<1>(s, index_q, ik_data, block_table, seq_lens, q_pos, scores, st);
      case 2: return launch_f32<2>(s, index_q, ik_data, block_table, seq_lens, q_pos, scores, st);
      case 4: return launch_f32<4>(s, index_q, ik_data, block_table, seq_lens, q_pos, scores, st);
      case 8: return launch_f32<8>(s, index_q, ik_data, block_table, seq_lens, q_pos, scores, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (s.G < 1 || s.G > 16) return hipErrorInvalidValue;
  IndexArgs x{};
  x.iq = static_cast<const uint16_t*>(index_q);
  x.ikd = static_cast<const uint8_t*>(ik_data);
  x.iks = static_cast<const uint8_t*>(ik_scales);
  x.bt = block_table;
  x.lens = seq_lens;
  x.qpos = q_pos;
  x.scores = scores;
  x.R = s.R;
  x.G = s.G;
  x.MB = s.MB;
  x.P = s.P;
  x.rows_per_wave = min(s.R, 16 / s.G);
  x.row_groups = (s.R + x.rows_per_wave - 1) / x.rows_per_wave;
  x.out_scale = s.index_scale * s.ik_scale;
  const int nseq = s.rows / s.R;
  x.B = nseq;
  x.share = s.share;
  if (s.share > 1 && s.R == 1) {  // shared scan (validated: R == 1)
    const int spw = share_per_wave(s.G);
    const int wgs_per_group = ((s.share + spw - 1) / spw + 3) / 4;
    const int groups = (nseq + s.share - 1) / s.share;
    const long wgs_per_block = (long)groups * wgs_per_group;
    const long total = wgs_per_block * ((s.MB + 7) / 8 * 8);  // j padded to a multiple of 8
    if (total > 0x7FFFFFFFL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)total);
    if (s.ik_dtype == kFP8)
      hipLaunchKernelGGL(index_shared_fp8_kernel, grid, dim3(256), 0, st, x, wgs_per_group,
                         (int)wgs_per_block);
    else
      hipLaunchKernelGGL(index_shared_nvfp4_kernel, grid, dim3(256), 0, st, x, wgs_per_group,
                         (int)wgs_per_block);
    return hipGetLastError();
  }
  const unsigned rgs = (unsigned)(nseq * x.row_groups);
  if (s.ik_dtype == kFP8) {
    constexpr int span = 4 * blocks_per_wave<kFP8>();
    hipLaunchKernelGGL(index_mfma_kernel<kFP8>, dim3((s.MB + span - 1) / span, rgs), dim3(256), 0,
                       st, x);
  } else {
    constexpr int span = 4 * blocks_per_wave<kNVFP4>();
    hipLaunchKernelGGL(index_mfma_kernel<kNVFP4>, dim3((s.MB + span - 1) / span, rgs), dim3(256),
                       0, st, x);
  }
  return hipGetLastError();
}

}  // namespace msa
