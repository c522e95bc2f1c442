// index_scores.hip -- lightning-indexer scoring + per-block max-pool.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer"): every cached key is scored by one index query per GQA group
// against one shared index-key head; the scores are max-pooled to one score
// per 128-token block.  Decode is HBM-bound: the scan reads 128 B per token
// (FP8) or 72 B (NVFP4), so these kernels stream each block once, coalesced,
// and keep all arithmetic in registers.
//
// Work decomposition: one wavefront per (query row, logical block); four
// wavefronts per workgroup take four consecutive blocks of the same row.
// Every load instruction of a wave reads 1 KB of consecutive bytes, and a
// block's loads are all issued before any arithmetic, to keep many bytes in
// flight per wave.  Blocks past a row's last visible key, and block-table
// entries outside the pool, produce -inf without touching the cache.
//
// Arithmetic: keys are converted exactly to bf16 (e4m3 and e2m1 values are
// bf16-representable) and multiplied with the bf16 index query by
// v_dot2c_f32_bf16: exact products, fp32 accumulation.  The positive score
// scale commutes with the max, so it is applied once per block.
#include "device.hpp"
#include "launch.hpp"

namespace msa {

// Optional side job of the first workgroup: zero n ints (the attention
// kernel's arrival counters, cleared here so msa_decode needs no extra launch).
struct ZeroArgs {
  int32_t* p;
  int n;
  __device__ __forceinline__ void run() const {
    if (p && blockIdx.x == 0 && blockIdx.y == 0)
      for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
  }
};

// -------------------------------------------------------------------------
// FP8 e4m3 index keys, bf16 index queries.
// Eight lanes share a token: lane l owns dims [16*(l%8), 16*(l%8)+16) of
// token l/8, so each 16-byte load instruction of the wave covers 8 tokens =
// 1 KB contiguously; the 16 KB block takes 16 such loads, all issued up front
// with the nontemporal hint (each byte is read exactly once).  A token's dot
// product is reduced over its 8 lanes in 3 DPP steps.
// -------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void index_fp8_kernel(
    const uint16_t* __restrict__ iq, const uint8_t* __restrict__ ik,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ qpos, float* __restrict__ scores, int R, int MB, int P,
    float out_scale, ZeroArgs za) {
  za.run();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.y, b = row / R;
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
  const uint4* src = reinterpret_cast<const uint4*>(ik + (size_t)pb * (kBlock * kDim)) + lane;
  uint4 raw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) raw[i] = load_stream(src + i * 64);
  // index query: dims [16c, 16c+16) of every group as bf16 pairs
  const int c = lane & 7;
  const uint4* qsrc = reinterpret_cast<const uint4*>(iq + (size_t)row * G * kDim) + c * 2;
  uint32_t qw[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 v = qsrc[g * 16 + i];
      qw[g][4 * i] = v.x;
      qw[g][4 * i + 1] = v.y;
      qw[g][4 * i + 2] = v.z;
      qw[g][4 * i + 3] = v.w;
    }
  }
  float m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = -INFINITY;
  const int tok0 = j * kBlock + (lane >> 3);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t kw[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 lo = fp8x2_to_bf16x2<false>(kw[w]);
      const bf16x2 hi = fp8x2_to_bf16x2<true>(kw[w]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        acc[g] = dot2_bf16(lo, as_bf16x2(qw[g][2 * w]), acc[g]);
        acc[g] = dot2_bf16(hi, as_bf16x2(qw[g][2 * w + 1]), acc[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      acc[g] += dpp<kQuadXor1>(acc[g]);
      acc[g] += dpp<kQuadXor2>(acc[g]);
      acc[g] += dpp<kHalfMirror>(acc[g]);
    }
    const bool valid = tok0 + i * 8 <= pos;
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = valid ? fmaxf(m[g], acc[g]) : m[g];
  }
  // max over the 8 token slots of the wave: lanes 8 apart hold other tokens
  float v = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = fmaxf(m[g], dpp<kRowRor8>(m[g]));
    x = fmaxf(x, shfl_xor(x, 16));
    x = fmaxf(x, shfl_xor(x, 32));
    if (lane == g) v = x;
  }
  if (lane < G) out[(size_t)lane * MB] = v * out_scale;
}

// -------------------------------------------------------------------------
// NVFP4 index keys (E2M1 data [BS][Di/2] + e4m3 scales [BS][Di/16]), bf16
// index queries.  The per-16 block scale is applied once per 16-element
// partial dot product; the tensor scale is folded into out_scale.
// -------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void index_nvfp4_kernel(
    const uint16_t* __restrict__ iq, const uint8_t* __restrict__ ikd,
    const uint8_t* __restrict__ iks, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ qpos,
    float* __restrict__ scores, int R, int MB, int P, float out_scale, ZeroArgs za) {
  za.run();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.y, b = row / R;
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
  const int c = lane & 3;
  // data: 16 tokens x 64 B = 1 KB per step; lane reads 16 B = dims [32c, 32c+32)
  const uint4* dsrc =
      reinterpret_cast<const uint4*>(ikd + (size_t)pb * (kBlock * kDim / 2)) + lane;
  // scales: 16 tokens x 8 B per step; lane reads the 2 scales of its 32 dims
  const uint16_t* ssrc = reinterpret_cast<const uint16_t*>(
                             iks + (size_t)pb * (kBlock * kDim / 16)) +
                         (lane >> 2) * 4 + c;
  uint4 raw[8];
  uint32_t sc[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    raw[s] = load_stream(dsrc + s * 64);
    sc[s] = __builtin_nontemporal_load(ssrc + s * 64);
  }
  const uint4* qsrc = reinterpret_cast<const uint4*>(iq + (size_t)row * G * kDim) + c * 4;
  uint32_t qw[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = qsrc[g * 16 + i];
      qw[g][4 * i] = v.x;
      qw[g][4 * i + 1] = v.y;
      qw[g][4 * i + 2] = v.z;
      qw[g][4 * i + 3] = v.w;
    }
  }
  float m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = -INFINITY;
  const int tok0 = j * kBlock + (lane >> 2);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint32_t dw[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
    const f32x2 scl = fp8x2_to_f32x2<false>(sc[s]);  // scales of dims [32c,+16), [32c+16,+16)
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float part[G];
#pragma unroll
      for (int g = 0; g < G; ++g) part[g] = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 2; ++ww) {
        const int w = half * 2 + ww;  // dword w holds dims 32c + 8w .. 8w+7
        const bf16x2 k0 = fp4x2_to_bf16x2<0>(dw[w]);
        const bf16x2 k1 = fp4x2_to_bf16x2<1>(dw[w]);
        const bf16x2 k2 = fp4x2_to_bf16x2<2>(dw[w]);
        const bf16x2 k3 = fp4x2_to_bf16x2<3>(dw[w]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          part[g] = dot2_bf16(k0, as_bf16x2(qw[g][4 * w]), part[g]);
          part[g] = dot2_bf16(k1, as_bf16x2(qw[g][4 * w + 1]), part[g]);
          part[g] = dot2_bf16(k2, as_bf16x2(qw[g][4 * w + 2]), part[g]);
          part[g] = dot2_bf16(k3, as_bf16x2(qw[g][4 * w + 3]), part[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = fmaf(scl[half], part[g], acc[g]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      acc[g] += dpp<kQuadXor1>(acc[g]);
      acc[g] += dpp<kQuadXor2>(acc[g]);
    }
    const bool valid = tok0 + s * 16 <= pos;
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = valid ? fmaxf(m[g], acc[g]) : m[g];
  }
  float v = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = fmaxf(m[g], dpp<kRowRor4>(m[g]));
    x = fmaxf(x, dpp<kRowRor8>(x));
    x = fmaxf(x, shfl_xor(x, 16));
    x = fmaxf(x, shfl_xor(x, 32));
    if (lane == g) v = x;
  }
  if (lane < G) out[(size_t)lane * MB] = v * out_scale;
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
    float out_scale, ZeroArgs za) {
  za.run();
  __shared__ float qs[G * kDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
static hipError_t launch_g(const Shape& s, const void* iq, const void* ikd, const void* iks,
                           const int32_t* bt, const int32_t* lens, const int32_t* qpos,
                           float* scores, hipStream_t st, int32_t* zero, int n_zero) {
  dim3 grid((s.MB + 3) / 4, s.rows), block(256);
  float out_scale = s.index_scale * s.ik_scale;
  const ZeroArgs za{zero, n_zero};
  if (s.ik_dtype == kFP8) {
    hipLaunchKernelGGL(index_fp8_kernel<G>, grid, block, 0, st, (const uint16_t*)iq,
                       (const uint8_t*)ikd, bt, lens, qpos, scores, s.R, s.MB, s.P, out_scale, za);
  } else if (s.ik_dtype == kNVFP4) {
    hipLaunchKernelGGL(index_nvfp4_kernel<G>, grid, block, 0, st, (const uint16_t*)iq,
                       (const uint8_t*)ikd, (const uint8_t*)iks, bt, lens, qpos, scores, s.R,
                       s.MB, s.P, out_scale, za);
  } else {
    hipLaunchKernelGGL(index_f32_kernel<G>, grid, block, 0, st, (const float*)iq,
                       (const float*)ikd, bt, lens, qpos, scores, s.R, s.MB, s.P, out_scale, za);
  }
  return hipGetLastError();
}

hipError_t launch_index_scores(const Shape& s, const void* index_q, const void* ik_data,
                               const void* ik_scales, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* q_pos,
                               float* scores, hipStream_t st, int32_t* zero, int n_zero) {
  switch (s.G) {
    case 1: return launch_g<1>(s, index_q, ik_data, ik_scales, block_table, seq_lens, q_pos, scores, st, zero, n_zero);
    case 2: return launch_g<2>(s, index_q, ik_data, ik_scales, block_table, seq_lens, q_pos, scores, st, zero, n_zero);
    case 4: return launch_g<4>(s, index_q, ik_data, ik_scales, block_table, seq_lens, q_pos, scores, st, zero, n_zero);
    case 8: return launch_g<8>(s, index_q, ik_data, ik_scales, block_table, seq_lens, q_pos, scores, st, zero, n_zero);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
