// cache_write.hip -- quantise new tokens into the paged caches (the insert
// half of a decode step: every new token's K and V for all groups and its
// index key go to their slot of the FP8 / NVFP4 / fp32 caches).
//
// Method: the caches the MSA kernels read (vLLM blog "Day-0 support for
// MiniMax-M3.1-Flash", sections "MSA primer" -- FP8 index keys, 128 B per
// token -- and the NVFP4 kernels section -- E2M1 values with one e4m3 scale
// per 16 elements and a per-tensor scale).  Each value is stored so that the
// read side's dequantisation (scale * code, or scale * e4m3(s) * e2m1(q))
// gives it back to the format's precision:
//   F32  : x / scale
//   FP8  : e4m3(x / scale), round to nearest even, saturating at +-448
//   NVFP4: per 16 elements s = e4m3(amax / (6 scale)), then
//          q = e2m1(x / (e4m3value(s) scale)) (0 when s is 0)
// where every arithmetic step is one correctly rounded binary32 operation,
// so the result is a function of the inputs alone.
//
// Work decomposition: one wavefront per (new token, plane): planes 0..G-1
// are the K rows of the G groups, G..2G-1 the V columns (V is stored
// transposed), 2G the index key.  Lane l takes dims 2l and 2l+1; an NVFP4
// group of 16 dims is 8 lanes, whose amax is a 3-step lane reduction.  V
// NVFP4 codes are nibbles shared with the neighbouring token's, written
// with atomic and/or on their 32-bit word so that two tokens' writes to one
// byte cannot interfere.
#include "device.hpp"
#include "launch.hpp"

namespace msa {

struct CacheWriteArgs {
  const int32_t* seq;
  const int32_t* pos;
  const void* k_new;
  const void* v_new;
  const void* ik_new;
  const int32_t* bt;
  uint8_t* kvd;
  uint8_t* kvs;
  uint8_t* ikd;
  uint8_t* iks;
  int n, B, G, MB, P;
  int kv_dtype, ik_dtype;
  int new_kv_f32, new_ik_f32;  // 1: new values are fp32, 0: bf16
  float k_scale, v_scale, ik_scale;
};

__device__ __forceinline__ float load_new(const void* base, size_t idx, int f32) {
  return f32 ? reinterpret_cast<const float*>(base)[idx]
             : bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

// e4m3 code of x: the hardware conversion rounds to nearest even; clamping
// to +-448 first gives the saturating encoding.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// E2M1 code of x: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even
// code (0, 1, 2 and 4 win their ties), saturating at 6, sign kept.
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float a = fabsf(x);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return c | (__float_as_uint(x) >> 31 << 3);
}

// The e4m3 value of code c (c < 0x7F: never NaN here).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return fp8x2_to_f32x2<false>(c)[0];
}

__global__ __launch_bounds__(64) void cache_write_kernel(CacheWriteArgs a) {
  const int lane = threadIdx.x;
  const int i = blockIdx.x, plane = blockIdx.y;
  const int b = a.seq[i], p = a.pos[i];
  if (b < 0 || b >= a.B || p < 0 || p >= a.MB * kBlock) return;  // out of range: skipped
  const int pb = a.bt[(size_t)b * a.MB + p / kBlock];
  if (pb < 0 || pb >= a.P) return;
  const int t = p % kBlock;
  const bool is_ik = plane == 2 * a.G;
  const int kv = plane < a.G ? 0 : 1, g = plane % a.G;
  const int dtype = is_ik ? a.ik_dtype : a.kv_dtype;
  const float scale = is_ik ? a.ik_scale : kv == 0 ? a.k_scale : a.v_scale;
  const int d0 = 2 * lane;
  float x0, x1;
  if (is_ik) {
    x0 = load_new(a.ik_new, (size_t)i * kDim + d0, a.new_ik_f32);
    x1 = load_new(a.ik_new, (size_t)i * kDim + d0 + 1, a.new_ik_f32);
  } else {
    const void* src = kv == 0 ? a.k_new : a.v_new;
    const size_t e = ((size_t)i * a.G + g) * kDim + d0;
    x0 = load_new(src, e, a.new_kv_f32);
    x1 = load_new(src, e + 1, a.new_kv_f32);
  }
  // plane base (in elements) and whether it is stored transposed ([d][t])
  const size_t base = is_ik ? (size_t)pb * kBlock * kDim
                            : (((size_t)pb * 2 + kv) * a.G + g) * (size_t)(kBlock * kDim);
  const bool transposed = !is_ik && kv == 1;
  uint8_t* data = is_ik ? a.ikd : a.kvd;
  uint8_t* scales = is_ik ? a.iks : a.kvs;

  if (dtype == kF32) {
    float* f = reinterpret_cast<float*>(data);
    const float q0 = x0 / scale, q1 = x1 / scale;
    if (transposed) {
      f[base + (size_t)d0 * kBlock + t] = q0;
      f[base + (size_t)(d0 + 1) * kBlock + t] = q1;
    } else {
      *reinterpret_cast<float2*>(f + base + (size_t)t * kDim + d0) = make_float2(q0, q1);
    }
  } else if (dtype == kFP8) {
    const uint32_t c = e4m3_pair(x0 / scale, x1 / scale);
    if (transposed) {
      data[base + (size_t)d0 * kBlock + t] = (uint8_t)c;
      data[base + (size_t)(d0 + 1) * kBlock + t] = (uint8_t)(c >> 8);
    } else {
      *reinterpret_cast<uint16_t*>(data + base + (size_t)t * kDim + d0) = (uint16_t)c;
    }
  } else {  // NVFP4: group of 16 dims = lanes 8k .. 8k+7
    float amax = fmaxf(fabsf(x0), fabsf(x1));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    const uint32_t s = e4m3_pair(amax / (6.0f * scale), 0.0f) & 0xFFu;
    const float sg = e4m3_value(s) * scale;
    const uint32_t q0 = sg == 0.0f ? 0u : e2m1_code(x0 / sg);
    const uint32_t q1 = sg == 0.0f ? 0u : e2m1_code(x1 / sg);
    const int grp = lane >> 3;
    if (!transposed) {  // [t][d/2] nibbles (even d low), scales [t][d/16]
      data[base / 2 + (size_t)t * (kDim / 2) + lane] = (uint8_t)(q0 | (q1 << 4));
      if ((lane & 7) == 0) scales[base / 16 + (size_t)t * (kDim / 16) + grp] = (uint8_t)s;
    } else {  // [d][t/2] nibbles (even t low), scales [d/16][t]
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const size_t byte = base / 2 + (size_t)(d0 + k) * (kBlock / 2) + t / 2;
        uint32_t* word = reinterpret_cast<uint32_t*>(data + (byte & ~(size_t)3));
        const int shift = (int)(byte & 3) * 8 + (t & 1) * 4;
        const uint32_t q = k == 0 ? q0 : q1;
        atomicAnd(word, ~(0xFu << shift));
        atomicOr(word, q << shift);
      }
      if ((lane & 7) == 0) scales[base / 16 + (size_t)grp * kBlock + t] = (uint8_t)s;
    }
  }
}

hipError_t launch_cache_write(const Shape& s, int num_tokens, const int32_t* token_seq,
                              const int32_t* token_pos, const void* k_new, const void* v_new,
                              const void* ik_new, const int32_t* block_table, void* kv_data,
                              void* kv_scales, void* ik_data, void* ik_scales, hipStream_t st) {
  if (num_tokens == 0) return hipSuccess;
  CacheWriteArgs a;
  a.seq = token_seq;
  a.pos = token_pos;
  a.k_new = k_new;
  a.v_new = v_new;
  a.ik_new = ik_new;
  a.bt = block_table;
  a.kvd = static_cast<uint8_t*>(kv_data);
  a.kvs = static_cast<uint8_t*>(kv_scales);
  a.ikd = static_cast<uint8_t*>(ik_data);
  a.iks = static_cast<uint8_t*>(ik_scales);
  a.n = num_tokens;
  a.B = s.rows / s.R;
  a.G = s.G;
  a.MB = s.MB;
  a.P = s.P;
  a.kv_dtype = s.kv_dtype;
  a.ik_dtype = s.ik_dtype;
  a.new_kv_f32 = s.q_dtype == kF32;
  a.new_ik_f32 = s.iq_dtype == kF32;
  a.k_scale = s.k_scale;
  a.v_scale = s.v_scale;
  a.ik_scale = s.ik_scale;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)num_tokens, (unsigned)(2 * s.G + 1)),
                     dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace msa
