// device.hpp -- gfx950 building blocks shared by the MSA kernels: number
// format conversions through the CDNA4 conversion instructions, DPP lane
// exchanges, and the MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kBlock = 128;  // tokens per KV block
constexpr int kDim = 128;    // head dim and index dim

// ---- number formats -------------------------------------------------------

// Two OCP e4m3 values (bytes 0,1 or, with HI, 2,3 of w) -> two bf16.  Every e4m3 value
// is exactly representable in bf16, so with a unit scale this is exact.
template <bool HI>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}
// Same into f16 (e4m3 range 2^-9..448 is inside f16's normal range: exact).
template <bool HI>
__device__ __forceinline__ f16x2 fp8x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}
// Two e4m3 -> two f32 (exact).
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}
// Two E2M1 values (byte `sel` of w, low nibble first) -> two bf16 (exact).
template <int SEL>
__device__ __forceinline__ bf16x2 fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// f32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// acc + a.x*b.x + a.y*b.y with fp32 accumulation (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

// Streaming 16-byte load with the nontemporal hint (data read exactly once).
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Row bookkeeping shared by the kernels: the last key a query row may see
// (keys t <= pos and t < seq_len, clamped to the block table's reach of
// MB blocks); negative when the row sees none.
__device__ __forceinline__ int row_last_key(const int32_t* lens, const int32_t* qpos, int row,
                                            int b, int MB) {
  const int last = min(lens[b], MB * kBlock) - 1;
  return qpos ? min(qpos[row], last) : last;
}

// ---- lane exchanges -------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kRowRor4 = 0x124;  // rotate right by 4 within 16 lanes
constexpr int kRowRor8 = 0x128;

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// ---- MFMA -----------------------------------------------------------------
// 16x16x32: A lane l holds A[l%16][8*(l/16)+e], B lane l holds B[8*(l/16)+e][l%16],
// D lane l holds D[4*(l/16)+i][l%16].
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace msa
