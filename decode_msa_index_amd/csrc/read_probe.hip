// read_probe.hip -- a measurement probe, not part of the MSA library: it
// reads the same 16 KB index-key blocks a decode scan reads, in the scan's
// order and with its access pattern (one wave per block, every load
// instruction 1 KB of consecutive bytes, all of a block's loads issued
// before anything waits), and does no arithmetic on them.  Its time per
// byte is the read bandwidth that this access pattern reaches, the ceiling
// the scan is measured against.  Built as its own library (libmsa_probe.so)
// for the benchmark's --calibrate-read mode.
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

}  // extern "C"
