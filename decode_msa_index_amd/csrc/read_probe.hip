// read_probe.hip -- measurement probes, not part of the MSA library.
//
// msa_probe_read_blocks reads the same 16 KB index-key blocks a decode scan
// reads, in the scan's order and with its access pattern (one wave per
// block, every load instruction 1 KB of consecutive bytes, all of a block's
// loads issued before anything waits), and does no arithmetic on them.  Its
// time per byte is the read bandwidth that this access pattern reaches, the
// ceiling the scan is measured against.
//
// msa_probe_read_kv reads what the one-wave attention launch reads: one
// wave per (row, group) walks the unit's selected blocks in selection order
// and reads each block's K and V planes (16 KB each, 32 loads of 1 KB issued
// together), again with no arithmetic: the floor of that kernel's time set
// by its K/V reads alone.
//
// msa_probe_read_records reads one record per block in the same one-wave,
// 1 KB-per-load pattern: `rec_bytes` at base + order[i] * rec_bytes, plus,
// optionally, `side_bytes` more at side + order[i] * side_bytes.  With 8 KB
// records and 1 KB side records it reads what the NVFP4 scan reads (E2M1
// data, e4m3 scales); with 9 KB records and no side records, the same bytes
// stored as one record per block.
//
// Built as its own library (libmsa_probe.so) for the benchmark's
// --calibrate-read mode.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Wave w of workgroup x takes blocks BPW * (4 x + w) + i (i < BPW): the
// blocks order[...] of 16 KB at base.  One word per wave goes to sink (the
// XOR of everything read), so the loads cannot be dropped.
template <int BPW>
__global__ __launch_bounds__(256) void read_blocks_kernel(const uint8_t* __restrict__ base,
                                                          const int32_t* __restrict__ order,
                                                          int nblocks, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int w = blockIdx.x * 4 + wave;
  const int b0 = w * BPW;
  if (b0 >= nblocks) return;
  u32x4v v[BPW][16];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int b = min(b0 + i, nblocks - 1);
    const u32x4v* src = reinterpret_cast<const u32x4v*>(base + (size_t)order[b] * 16384) + lane;
#pragma unroll
    for (int k = 0; k < 16; ++k) v[i][k] = __builtin_nontemporal_load(src + k * 64);
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
#pragma unroll
    for (int k = 0; k < 16; ++k) x ^= v[i][k].x ^ v[i][k].y ^ v[i][k].z ^ v[i][k].w;
  }
  // reduce over the wave first: every lane's loads then feed the one store
  // (a value only lane 0 used would let the compiler move the loads under
  // the lane-0 branch, and read 16 bytes per load instead of 1 KB)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if (lane == 0) sink[w] = x;
}

// One wave per unit u = row * G + g: the K plane (p, 0, g) and the V plane
// (p, 1, g) of every selected block, p = bt[b][j] for j = topk[u][e].
// Entries outside [0, MB) and table entries outside [0, P) are skipped.
__global__ __launch_bounds__(64) void read_kv_kernel(const uint8_t* __restrict__ kv,
                                                     const int32_t* __restrict__ topk,
                                                     const int32_t* __restrict__ bt, int K, int G,
                                                     int R, int MB, int P,
                                                     uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  const int u = blockIdx.x, row = u / G, g = u % G, b = row / R;
  uint32_t x = 0;
  for (int e = 0; e < K; ++e) {
    const int j = topk[(size_t)u * K + e];
    if (j < 0 || j >= MB) continue;
    const int p = bt[(size_t)b * MB + j];
    if (p < 0 || p >= P) continue;
    const u32x4v* kp = reinterpret_cast<const u32x4v*>(kv + (((size_t)p * 2 + 0) * G + g) * 16384) + lane;
    const u32x4v* vp = reinterpret_cast<const u32x4v*>(kv + (((size_t)p * 2 + 1) * G + g) * 16384) + lane;
    u32x4v v[32];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      v[k] = kp[k * 64];
      v[16 + k] = vp[k * 64];
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if (lane == 0) sink[u] = x;
}

// One wave per block: R 1 KB chunks of the record, then S of the side record
// (R <= 16, S <= 1), all issued before any is used.
template <int R, int S>
__global__ __launch_bounds__(256) void read_records_kernel(const uint8_t* __restrict__ base,
                                                           const uint8_t* __restrict__ side,
                                                           const int32_t* __restrict__ order,
                                                           int nblocks, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int w = blockIdx.x * 4 + wave;
  if (w >= nblocks) return;
  const size_t b = (size_t)order[w];
  const u32x4v* src = reinterpret_cast<const u32x4v*>(base + b * (R * 1024)) + lane;
  u32x4v v[R + S];
#pragma unroll
  for (int k = 0; k < R; ++k) v[k] = __builtin_nontemporal_load(src + k * 64);
  if constexpr (S > 0) {
    const u32x4v* ssrc = reinterpret_cast<const u32x4v*>(side + b * (S * 1024)) + lane;
#pragma unroll
    for (int k = 0; k < S; ++k) v[R + k] = __builtin_nontemporal_load(ssrc + k * 64);
  }
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < R + S; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if (lane == 0) sink[w] = x;
}

}  // namespace

extern "C" {

// Reads nblocks blocks of 16 KB: block i is base + order[i] * 16384.
// blocks_per_wave: 1, 2 or 4 (all of a wave's loads in flight together).
// sink: one uint32 per wave (ceil(nblocks / blocks_per_wave) words).
hipError_t msa_probe_read_blocks(const void* base, const int32_t* order, int nblocks,
                                 int blocks_per_wave, uint32_t* sink, void* stream) {
  if (nblocks <= 0) return hipSuccess;
  const int waves = (nblocks + blocks_per_wave - 1) / blocks_per_wave;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  const uint8_t* b = static_cast<const uint8_t*>(base);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (blocks_per_wave) {
    case 1: hipLaunchKernelGGL(read_blocks_kernel<1>, grid, block, 0, st, b, order, nblocks, sink); break;
    case 2: hipLaunchKernelGGL(read_blocks_kernel<2>, grid, block, 0, st, b, order, nblocks, sink); break;
    case 4: hipLaunchKernelGGL(read_blocks_kernel<4>, grid, block, 0, st, b, order, nblocks, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Reads nblocks records: block i is rec_kib KB at base + order[i] * rec_kib
// KB, plus side_kib KB at side + order[i] * side_kib KB.  Supported:
// (rec_kib, side_kib) = (8, 1), (8, 0), (9, 0).  sink: one uint32 per block.
hipError_t msa_probe_read_records(const void* base, const void* side, const int32_t* order,
                                  int nblocks, int rec_kib, int side_kib, uint32_t* sink,
                                  void* stream) {
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)((nblocks + 3) / 4)), block(256);
  const uint8_t* b = static_cast<const uint8_t*>(base);
  const uint8_t* sd = static_cast<const uint8_t*>(side);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (rec_kib == 8 && side_kib == 1) {
    if (!sd) return hipErrorInvalidValue;
    hipLaunchKernelGGL((read_records_kernel<8, 1>), grid, block, 0, st, b, sd, order, nblocks, sink);
  } else if (rec_kib == 8 && side_kib == 0) {
    hipLaunchKernelGGL((read_records_kernel<8, 0>), grid, block, 0, st, b, sd, order, nblocks, sink);
  } else if (rec_kib == 9 && side_kib == 0) {
    hipLaunchKernelGGL((read_records_kernel<9, 0>), grid, block, 0, st, b, sd, order, nblocks, sink);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Reads the K and V planes (16 KB each, FP8 cache) of every selected block of
// units (row, group) pairs: kv = [P][2][G][16 KB], topk = [units][K], bt =
// [rows / R][MB].  sink: one uint32 per unit.
hipError_t msa_probe_read_kv(const void* kv, const int32_t* topk, const int32_t* bt, int units,
                             int K, int G, int R, int MB, int P, uint32_t* sink, void* stream) {
  if (units <= 0) return hipSuccess;
  if (K < 1 || G < 1 || R < 1 || MB < 1 || P < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kv_kernel, dim3((unsigned)units), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(kv), topk, bt,
                     K, G, R, MB, P, sink);
  return hipGetLastError();
}

}  // extern "C"
