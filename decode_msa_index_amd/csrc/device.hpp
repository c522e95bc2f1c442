// device.hpp -- gfx950 building blocks shared by the MSA kernels: number
// format conversions through the CDNA4 conversion instructions, DPP lane
// exchanges, and the MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: loops and addresses derived from it stay scalar.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

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

// ---- 8-element conversions for MFMA operands -------------------------------

typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef _Float16 f16x4 __attribute__((__vector_size__(4 * sizeof(_Float16))));

__device__ __forceinline__ bf16x8 cat(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x8 cat(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  const f16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const f16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 8 e4m3 bytes (w0: elements 0..3, w1: 4..7) -> bf16x8 / f16x8, exact.
__device__ __forceinline__ bf16x8 fp8x8_bf16(uint32_t w0, uint32_t w1) {
  return cat(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
             fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
}
__device__ __forceinline__ f16x8 fp8x8_f16(uint32_t w0, uint32_t w1) {
  return cat(fp8x2_to_f16x2<false>(w0), fp8x2_to_f16x2<true>(w0),
             fp8x2_to_f16x2<false>(w1), fp8x2_to_f16x2<true>(w1));
}

// upper halves of two f32 -> one bf16x2 word (exact when the low halves are 0)
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 8 E2M1 values (nibbles of w, element 2b in the low nibble of byte b) times
// one e4m3 block scale -> bf16x8.  The product of an e4m3 and an E2M1 value
// has at most 6 significant bits and lies in [2^-10, 2688]: exact in fp32 and
// in bf16.
__device__ __forceinline__ bf16x8 nvfp4x8_bf16(uint32_t w, float scale) {
  const f32x2 a = fp4x2_to_f32x2<0>(w), b = fp4x2_to_f32x2<1>(w);
  const f32x2 c = fp4x2_to_f32x2<2>(w), d = fp4x2_to_f32x2<3>(w);
  uint4 r;
  r.x = pack_hi16(a[0] * scale, a[1] * scale);
  r.y = pack_hi16(b[0] * scale, b[1] * scale);
  r.z = pack_hi16(c[0] * scale, c[1] * scale);
  r.w = pack_hi16(d[0] * scale, d[1] * scale);
  return __builtin_bit_cast(bf16x8, r);
}

// 8 E2M1 values, element e scaled by e4m3 byte e of (s0, s1) -> f16x8 (exact:
// same bound as above, inside f16's normal range).
__device__ __forceinline__ f16x8 nvfp4x8_f16(uint32_t w, uint32_t s0, uint32_t s1) {
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return cat(v0 * fp8x2_to_f16x2<false>(s0), v1 * fp8x2_to_f16x2<true>(s0),
             v2 * fp8x2_to_f16x2<false>(s1), v3 * fp8x2_to_f16x2<true>(s1));
}

// 8 E2M1 values (nibbles of w, element 2b in the low nibble of byte b) times
// one f16 block scale given in both halves of s -> f16x8 (exact, as above).
__device__ __forceinline__ f16x8 nvfp4x8_f16s(uint32_t w, f16x2 s) {
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return cat(v0 * s, v1 * s, v2 * s, v3 * s);
}

// ---- lane exchanges -------------------------------------------------------

// Keeps the compiler from moving LDS accesses across this point; the
// hardware already executes a wave's LDS operations in order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// Value of lane (lane ^ J).  J = 1, 2, 8 are single DPP moves (quad
// permutes, rotate a 16-lane row by 8); J = 4 takes the lane 4 up or down
// with two DPP row shifts; 16 and 32 use the CDNA4 row-swap instructions
// (v_permlane16_swap / v_permlane32_swap with both operands = v: the first
// result holds the even rows / lower half, the second the odd rows / upper
// half).
template <int J>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);  // row_shl:4
    const int dn = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 16) ? r[0] : r[1]);
  } else {
    static_assert(J == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 32) ? r[0] : r[1]);
  }
}

template <int J>
__device__ __forceinline__ float lane_xor_f(float v) {
  return __builtin_bit_cast(float, lane_xor<J>(__builtin_bit_cast(int, v)));
}


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
