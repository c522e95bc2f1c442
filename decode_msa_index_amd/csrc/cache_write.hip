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
// Work decomposition: lane l of a wavefront quantises dims 2l and 2l+1 of
// one new token's plane: planes 0..G-1 are the K rows of the G groups,
// G..2G-1 the V columns (V is stored transposed), 2G the index key; an
// NVFP4 group of 16 dims is 8 lanes, whose amax is a 3-step lane
// reduction.  Short token lists take one wave per (token, plane)
// (cache_write_token_kernel); long ones take workgroups of 16 consecutive
// list entries, which write aligned runs of consecutive positions (a
// prefill chunk) a V dim row at a time (cache_write_kernel).  V NVFP4 codes
// written token by token are nibbles shared with the neighbouring token's,
// written with atomic and/or on their 32-bit word so that two tokens'
// writes to one byte cannot interfere.
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

// The codes of dims 2 lane and 2 lane + 1 of one token's plane: F32 values
// (as bits), FP8 bytes, or E2M1 nibbles plus the e4m3 scale of their group of
// 16 dims (lanes 8k .. 8k+7, whose amax is a 3-step lane reduction).
struct PairCodes {
  uint32_t c0, c1, s;
};
__device__ __forceinline__ PairCodes quant_pair(int dtype, float x0, float x1, float scale) {
  PairCodes q{0u, 0u, 0u};
  if (dtype == kF32) {
    q.c0 = __float_as_uint(x0 / scale);
    q.c1 = __float_as_uint(x1 / scale);
  } else if (dtype == kFP8) {
    const uint32_t c = e4m3_pair(x0 / scale, x1 / scale);
    q.c0 = c & 0xFFu;
    q.c1 = c >> 8;
  } else {
    float amax = fmaxf(fabsf(x0), fabsf(x1));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    q.s = e4m3_pair(amax / (6.0f * scale), 0.0f) & 0xFFu;
    const float sg = e4m3_value(q.s) * scale;
    q.c0 = sg == 0.0f ? 0u : e2m1_code(x0 / sg);
    q.c1 = sg == 0.0f ? 0u : e2m1_code(x1 / sg);
  }
  return q;
}

// Plane base (in elements) of (physical block pb, plane): planes 0..G-1 the
// K rows, G..2G-1 the V columns (stored transposed), 2G the index key.
__device__ __forceinline__ size_t plane_base(const CacheWriteArgs& a, int pb, int plane) {
  if (plane == 2 * a.G) return (size_t)pb * kBlock * kDim;
  const int kv = plane < a.G ? 0 : 1, g = plane % a.G;
  return (((size_t)pb * 2 + kv) * a.G + g) * (size_t)(kBlock * kDim);
}

// Dims 2 lane, 2 lane + 1 of new token i's plane as raw bits: one 8-byte
// (f32) or 4-byte (bf16 pair, in .x) load; values() converts them where they
// are used, so that a wave's loads of all planes can be in flight together.
template <bool F32>
__device__ __forceinline__ uint2 load_new_pair(const void* base, size_t idx) {
  if constexpr (F32) return *reinterpret_cast<const uint2*>(reinterpret_cast<const float*>(base) + idx);
  return make_uint2(*reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(base) + idx),
                    0u);
}
template <bool F32>
__device__ __forceinline__ float2 values(uint2 r) {
  if constexpr (F32) return make_float2(__uint_as_float(r.x), __uint_as_float(r.y));
  return make_float2(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u));
}
template <bool KV_F32, bool IK_F32>
__device__ __forceinline__ uint2 load_pair(const CacheWriteArgs& a, int i, int plane, int lane) {
  const int d0 = 2 * lane;
  if (plane == 2 * a.G) return load_new_pair<IK_F32>(a.ik_new, (size_t)i * kDim + d0);
  const void* src = plane < a.G ? a.k_new : a.v_new;
  return load_new_pair<KV_F32>(src, ((size_t)i * a.G + plane % a.G) * kDim + d0);
}

// A new token's slot: its physical block and row, or pb = -1 when the
// token's sequence, position or table entry is out of range (skipped).
struct Slot {
  int pb, t;
};

// One token's plane, one wave (lane l: dims 2l, 2l+1, values x), stored in
// place at row t of physical block pb.
__device__ __forceinline__ void store_token_plane(const CacheWriteArgs& a, int pb, int t,
                                                  int plane, int lane, float2 x) {
  const bool is_ik = plane == 2 * a.G;
  const int kv = plane < a.G ? 0 : 1;
  const int dtype = is_ik ? a.ik_dtype : a.kv_dtype;
  const float scale = is_ik ? a.ik_scale : kv == 0 ? a.k_scale : a.v_scale;
  const int d0 = 2 * lane;
  const PairCodes q = quant_pair(dtype, x.x, x.y, scale);
  const size_t base = plane_base(a, pb, plane);
  const bool transposed = !is_ik && kv == 1;
  uint8_t* data = is_ik ? a.ikd : a.kvd;
  uint8_t* scales = is_ik ? a.iks : a.kvs;

  if (dtype == kF32) {
    float* f = reinterpret_cast<float*>(data);
    if (transposed) {
      f[base + (size_t)d0 * kBlock + t] = __uint_as_float(q.c0);
      f[base + (size_t)(d0 + 1) * kBlock + t] = __uint_as_float(q.c1);
    } else {
      *reinterpret_cast<float2*>(f + base + (size_t)t * kDim + d0) =
          make_float2(__uint_as_float(q.c0), __uint_as_float(q.c1));
    }
  } else if (dtype == kFP8) {
    if (transposed) {
      data[base + (size_t)d0 * kBlock + t] = (uint8_t)q.c0;
      data[base + (size_t)(d0 + 1) * kBlock + t] = (uint8_t)q.c1;
    } else {
      *reinterpret_cast<uint16_t*>(data + base + (size_t)t * kDim + d0) =
          (uint16_t)(q.c0 | (q.c1 << 8));
    }
  } else {  // NVFP4: group of 16 dims = lanes 8k .. 8k+7
    const int grp = lane >> 3;
    if (!transposed) {  // [t][d/2] nibbles (even d low), scales [t][d/16]
      data[base / 2 + (size_t)t * (kDim / 2) + lane] = (uint8_t)(q.c0 | (q.c1 << 4));
      if ((lane & 7) == 0) scales[base / 16 + (size_t)t * (kDim / 16) + grp] = (uint8_t)q.s;
    } else {  // [d][t/2] nibbles (even t low), scales [d/16][t]
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const size_t byte = base / 2 + (size_t)(d0 + k) * (kBlock / 2) + t / 2;
        uint32_t* word = reinterpret_cast<uint32_t*>(data + (byte & ~(size_t)3));
        const int shift = (int)(byte & 3) * 8 + (t & 1) * 4;
        const uint32_t c = k == 0 ? q.c0 : q.c1;
        atomicAnd(word, ~(0xFu << shift));
        atomicOr(word, c << shift);
      }
      if ((lane & 7) == 0) scales[base / 16 + (size_t)grp * kBlock + t] = (uint8_t)q.s;
    }
  }
}

// Short lists (a decode step's few new tokens): one wave per (token, plane)
// over the whole chip.  A token's transposed V values land a block's row
// apart, 64 cache lines per store instruction; spread over many compute
// units those stores run in parallel.  Grid (tokens, 2G + 1).
template <bool KV_F32, bool IK_F32>
__global__ __launch_bounds__(64) void cache_write_token_kernel(CacheWriteArgs a) {
  const int lane = threadIdx.x, i = blockIdx.x, plane = blockIdx.y;
  const int b = a.seq[i], p = a.pos[i];
  if (b < 0 || b >= a.B || p < 0 || p >= a.MB * kBlock) return;  // out of range: skipped
  const int pb = a.bt[(size_t)b * a.MB + p / kBlock];
  if (pb < 0 || pb >= a.P) return;
  const uint2 r = load_pair<KV_F32, IK_F32>(a, i, plane, lane);
  const float2 v = plane == 2 * a.G ? values<IK_F32>(r) : values<KV_F32>(r);
  store_token_plane(a, pb, p % kBlock, plane, lane, v);
}

// Long lists (a prefill chunk's tokens): a workgroup takes kRun consecutive
// entries of the token list, a wave each; every wave issues the loads of all
// its token's planes first.  K and index-key rows are row-major, so each is
// one contiguous store per wave.
// V columns are stored transposed ([d][t]): written one token at a time
// they are single bytes (FP8) or nibbles a block's row apart.  When the
// workgroup's entries form an aligned run -- one sequence, positions p0 ..
// p0 + kRun - 1 with p0 % kRun == 0, so inside one block -- the V codes of
// each group meet in LDS and every dim row is written with one contiguous
// store (FP8 16 bytes, NVFP4 8 bytes of nibbles plus 16-byte scale rows, f32
// 64 bytes); the run owns those bytes whole, so no atomics are needed.
// Otherwise each wave writes its token's V too.
constexpr int kRun = 16;
constexpr int kShortList = 512;  // lists shorter than this take cache_write_token_kernel

template <int G, bool KV_F32, bool IK_F32>
__global__ __launch_bounds__(64 * kRun) void cache_write_kernel(CacheWriteArgs a) {
  __shared__ uint32_t codes[kRun][kDim];        // per token and dim: F32 bits / FP8 byte / nibble
  __shared__ uint32_t gscale[kRun][kDim / 16];  // NVFP4: per token and group of 16 dims
  const int lane = threadIdx.x & 63, w = wave_id();
  const int i0 = blockIdx.x * kRun, i = i0 + w;
  // lane e < kRun: list entry i0 + e's sequence and position (one load for
  // the whole workgroup's decisions)
  int sq = -1, ps = -1;
  if (lane < kRun && i0 + lane < a.n) {
    sq = a.seq[i0 + lane];
    ps = a.pos[i0 + lane];
  }
  // are entries i0 .. i0 + kRun - 1 an aligned run of one sequence in one block?
  const int s0 = __builtin_amdgcn_readfirstlane(sq), p0 = __builtin_amdgcn_readfirstlane(ps);
  const bool mine = lane >= kRun || (i0 + lane < a.n && sq == s0 && ps == p0 + lane);
  const bool cand = __ballot(!mine) == 0 && s0 >= 0 && s0 < a.B && p0 >= 0 &&
                    p0 % kRun == 0 && p0 + kRun <= a.MB * kBlock;
  // this wave's token (entry w) and its slot; the run's table entry is
  // loaded alongside
  const int b = __builtin_amdgcn_readlane(sq, w), p = __builtin_amdgcn_readlane(ps, w);
  const bool ok = i < a.n && b >= 0 && b < a.B && p >= 0 && p < a.MB * kBlock;
  const int e = ok ? a.bt[(size_t)b * a.MB + p / kBlock] : -1;
  const int rpb = cand ? a.bt[(size_t)s0 * a.MB + p0 / kBlock] : -1;
  const bool run = rpb >= 0 && rpb < a.P;  // the same decision in every wave
  const Slot sl{(e >= 0 && e < a.P) ? e : -1, p % kBlock};

  // this wave's token: all planes' values loaded first
  constexpr int NP = 2 * G + 1;
  uint2 x[NP];
  if (sl.pb >= 0) {
#pragma unroll
    for (int pl = 0; pl < NP; ++pl) x[pl] = load_pair<KV_F32, IK_F32>(a, i, pl, lane);
  }
  if (sl.pb >= 0) {
#pragma unroll
    for (int pl = 0; pl < NP; ++pl) {
      const bool v_plane = pl >= G && pl < 2 * G;
      if (!(run && v_plane)) {
        const float2 v = pl == 2 * G ? values<IK_F32>(x[pl]) : values<KV_F32>(x[pl]);
        store_token_plane(a, sl.pb, sl.t, pl, lane, v);
      }
    }
  }
  if (!run) return;

  // the run's V, one group at a time through LDS
  const int tid = threadIdx.x, t0 = p0 % kBlock;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float2 v = values<KV_F32>(x[G + g]);
    const PairCodes q = quant_pair(a.kv_dtype, v.x, v.y, a.v_scale);
    codes[w][2 * lane] = q.c0;
    codes[w][2 * lane + 1] = q.c1;
    if ((lane & 7) == 0) gscale[w][lane >> 3] = q.s;
    __syncthreads();
    const size_t base = plane_base(a, rpb, G + g);
    if (a.kv_dtype == kF32) {
      if (tid < kDim) {
        float4* f = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.kvd) + base +
                                              (size_t)tid * kBlock + t0);
#pragma unroll
        for (int k = 0; k < kRun / 4; ++k)
          f[k] = make_float4(__uint_as_float(codes[4 * k][tid]),
                             __uint_as_float(codes[4 * k + 1][tid]),
                             __uint_as_float(codes[4 * k + 2][tid]),
                             __uint_as_float(codes[4 * k + 3][tid]));
      }
    } else if (a.kv_dtype == kFP8) {
      if (tid < kDim) {
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          wd[k] = codes[4 * k][tid] | (codes[4 * k + 1][tid] << 8) |
                  (codes[4 * k + 2][tid] << 16) | (codes[4 * k + 3][tid] << 24);
        *reinterpret_cast<uint4*>(a.kvd + base + (size_t)tid * kBlock + t0) =
            make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    } else {
      if (tid < kDim) {  // [d][t/2]: byte k of the run = tokens 2k (low nibble), 2k + 1
        uint32_t wd[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          wd[h] = 0u;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            wd[h] |= (codes[8 * h + 2 * k][tid] | (codes[8 * h + 2 * k + 1][tid] << 4)) << (8 * k);
        }
        *reinterpret_cast<uint2*>(a.kvd + base / 2 + (size_t)tid * (kBlock / 2) + t0 / 2) =
            make_uint2(wd[0], wd[1]);
      } else if (tid < kDim + kDim / 16) {  // [d/16][t]: the run's 16 scales of group grp
        const int grp = tid - kDim;
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          wd[k] = gscale[4 * k][grp] | (gscale[4 * k + 1][grp] << 8) |
                  (gscale[4 * k + 2][grp] << 16) | (gscale[4 * k + 3][grp] << 24);
        *reinterpret_cast<uint4*>(a.kvs + base / 16 + (size_t)grp * kBlock + t0) =
            make_uint4(wd[0], wd[1], wd[2], wd[3]);
      }
    }
    __syncthreads();  // the LDS is reused by the next group
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
  if (num_tokens < kShortList) {
    const dim3 tgrid((unsigned)num_tokens, (unsigned)(2 * s.G + 1));
    if (a.new_kv_f32 && a.new_ik_f32)
      hipLaunchKernelGGL((cache_write_token_kernel<true, true>), tgrid, dim3(64), 0, st, a);
    else if (a.new_kv_f32)
      hipLaunchKernelGGL((cache_write_token_kernel<true, false>), tgrid, dim3(64), 0, st, a);
    else if (a.new_ik_f32)
      hipLaunchKernelGGL((cache_write_token_kernel<false, true>), tgrid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((cache_write_token_kernel<false, false>), tgrid, dim3(64), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((num_tokens + kRun - 1) / kRun)), block(64 * kRun);
#define MSA_CW_LAUNCH(GV)                                                              \
  if (a.new_kv_f32 && a.new_ik_f32)                                                    \
    hipLaunchKernelGGL((cache_write_kernel<GV, true, true>), grid, block, 0, st, a);   \
  else if (a.new_kv_f32)                                                               \
    hipLaunchKernelGGL((cache_write_kernel<GV, true, false>), grid, block, 0, st, a);  \
  else if (a.new_ik_f32)                                                               \
    hipLaunchKernelGGL((cache_write_kernel<GV, false, true>), grid, block, 0, st, a);  \
  else                                                                                 \
    hipLaunchKernelGGL((cache_write_kernel<GV, false, false>), grid, block, 0, st, a);
  switch (s.G) {
    case 1: MSA_CW_LAUNCH(1) break;
    case 2: MSA_CW_LAUNCH(2) break;
    case 4: MSA_CW_LAUNCH(4) break;
    case 8: MSA_CW_LAUNCH(8) break;
    default: return hipErrorInvalidValue;
  }
#undef MSA_CW_LAUNCH
  return hipGetLastError();
}

}  // namespace msa
