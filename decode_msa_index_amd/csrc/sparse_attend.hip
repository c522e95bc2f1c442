// sparse_attend.hip -- exact GQA attention over the selected KV blocks.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer" and Figure 1): every query head of a GQA group attends exactly the
// group's selected blocks, at most k*128 keys.  The attention itself is
// ordinary softmax attention, run split-K over the selected blocks (the API
// reference of MiniMaxM3SparseAttention._run_attention describes split-K
// attend kernels that read per-request metadata).
//
// Grid: one single-wave workgroup per (row, group, selected block).  Each
// computes, for the group's (up to 16) heads and the block's 128 keys,
//   S^T = K Q^T            v_mfma_f32_16x16x32_bf16  (K e4m3/e2m1 -> bf16 exact)
//   P   = exp2(S*scale - m) in fp32, rounded to f16 for the next product
//   O   = P V              v_mfma_f32_16x16x32_f16   (V e4m3/e2m1 -> f16 exact)
// and stores (m, l, O) as a partial.  The last workgroup of a (row, group) to
// finish -- found with a device-scope counter -- merges the partials, scales
// by v_scale / l and writes the output, then zeroes the counter.
//
// Operand layout.  The contraction order inside an MFMA is free as long as
// both operands agree, so the key order of the S^T tiles is chosen to make
// every global load contiguous: tile u (0..7) row m holds key
//   kappa(u, m) = 32*(m/4) + 8*(u/2) + 4*(u%2) + m%4,
// which puts, for PV chunk c, keys 32*(l/16) + 8*c + 0..7 into lane l's
// eight A elements -- exactly the 8 consecutive bytes of a V^T row that the
// B operand needs (V is stored transposed, [d][t], for this).
#include "device.hpp"
#include "launch.hpp"

namespace msa {

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// Split bookkeeping shared by the kernels: publish this split's partial, and
// if it is the last one of its (row, group), merge all of them.
// ---------------------------------------------------------------------------
struct AttendArgs {
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* qpos;
  const int32_t* topk;
  void* out;
  float* lse;
  int32_t* counters;
  float* part_o;
  float* part_ml;
  int R, H, G, hpg, MB, K;
  float scale_log2;  // sm_scale * k_scale * log2(e)
  float v_scale;
  int out_f32;
};

__device__ __forceinline__ void finish_split(const AttendArgs& a, int u, int count) {
  const int lane = threadIdx.x;
  __threadfence();
  int prev = 0;
  if (lane == 0) prev = atomicAdd(&a.counters[u], 1);
  prev = __shfl(prev, 0, 64);
  if (prev != count - 1) return;
  __threadfence();
  const int row = u / a.G, g = u % a.G;
  const float* po = a.part_o + (size_t)u * a.K * (kHeadsPad * 128);
  const float* pml = a.part_ml + (size_t)u * a.K * (kHeadsPad * 2);
  for (int h = 0; h < a.hpg; ++h) {
    float ms = -INFINITY, ls = 0.0f;
    if (lane < count) {
      ms = __builtin_nontemporal_load(pml + (size_t)lane * (kHeadsPad * 2) + 2 * h);
      ls = __builtin_nontemporal_load(pml + (size_t)lane * (kHeadsPad * 2) + 2 * h + 1);
    }
    const float M = wave_max(ms);
    const float w = lane < count ? exp2f(ms - M) : 0.0f;
    const float L = wave_sum(w * ls);
    float o0 = 0.0f, o1 = 0.0f;
    for (int s = 0; s < count; ++s) {
      const float ws = __shfl(w, s, 64);
      const float* src = po + (size_t)s * (kHeadsPad * 128) + h * 128;
      o0 = fmaf(ws, __builtin_nontemporal_load(src + lane), o0);
      o1 = fmaf(ws, __builtin_nontemporal_load(src + lane + 64), o1);
    }
    const float f = a.v_scale / L;
    const size_t orow = ((size_t)row * a.H + (size_t)g * a.hpg + h) * 128;
    if (a.out_f32) {
      float* o = reinterpret_cast<float*>(a.out) + orow;
      o[lane] = o0 * f;
      o[lane + 64] = o1 * f;
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + orow;
      o[lane] = f32_to_bf16(o0 * f);
      o[lane + 64] = f32_to_bf16(o1 * f);
    }
    if (a.lse && lane == 0)
      a.lse[(size_t)row * a.H + (size_t)g * a.hpg + h] = (M + log2f(L)) * 0.69314718055994531f;
  }
  if (lane == 0) a.counters[u] = 0;
}

// Common prologue: which block this workgroup takes, or -1 if none.
struct SplitInfo {
  int u, row, g, b, count, j, pb, nvalid;
};
__device__ __forceinline__ bool split_info(const AttendArgs& a, SplitInfo& si) {
  si.u = blockIdx.y;
  si.row = si.u / a.G;
  si.g = si.u % a.G;
  si.b = si.row / a.R;
  const int pos = a.qpos ? a.qpos[si.row] : a.lens[si.b] - 1;
  const int rb = pos / kBlock;
  si.count = min(a.K, rb + 1);
  if ((int)blockIdx.x >= si.count) return false;
  si.j = a.topk[(size_t)si.u * a.K + blockIdx.x];
  if (si.j < 0 || si.j > rb) {  // malformed selection: contribute nothing
    si.pb = -1;
    si.nvalid = 0;
    return true;
  }
  si.pb = a.bt[(size_t)si.b * a.MB + si.j];
  si.nvalid = min(kBlock, pos - si.j * kBlock + 1);
  return true;
}

__device__ __forceinline__ void store_empty_partial(const AttendArgs& a, const SplitInfo& si) {
  const int lane = threadIdx.x;
  float* pml = a.part_ml + ((size_t)si.u * a.K + blockIdx.x) * (kHeadsPad * 2);
  if (lane < kHeadsPad) {
    pml[2 * lane] = -INFINITY;
    pml[2 * lane + 1] = 0.0f;
  }
  float* po = a.part_o + ((size_t)si.u * a.K + blockIdx.x) * (kHeadsPad * 128);
  for (int i = lane; i < kHeadsPad * 128; i += 64) po[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// FP8 / NVFP4 cache, bf16 queries: MFMA tiles.
// ---------------------------------------------------------------------------
template <int KV>
__global__ __launch_bounds__(64) void attend_mfma_kernel(const uint16_t* __restrict__ q,
                                                         const uint8_t* __restrict__ kvd,
                                                         const uint8_t* __restrict__ kvs,
                                                         AttendArgs a) {
  SplitInfo si;
  if (!split_info(a, si)) return;
  const int lane = threadIdx.x;
  if (si.pb < 0) {
    store_empty_partial(a, si);
    finish_split(a, si.u, si.count);
    return;
  }
  const int n = lane & 15, qd = lane >> 4;
  const size_t kplane = ((size_t)si.pb * 2 + 0) * a.G + si.g;
  const size_t vplane = ((size_t)si.pb * 2 + 1) * a.G + si.g;

  // ---- loads: K rows kappa(u, n), V^T rows dt*16+n; 32 dims / tokens each ----
  uint4 kraw[16], vraw[16];
  uint32_t ksc[8];
  uint4 vsc[16];
  if constexpr (KV == kFP8) {
    const uint8_t* kb = kvd + kplane * (kBlock * kDim);
    const uint8_t* vb = kvd + vplane * (kBlock * kDim);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kappa = 32 * (n >> 2) + 8 * (u >> 1) + 4 * (u & 1) + (n & 3);
      const uint4* p = reinterpret_cast<const uint4*>(kb + kappa * kDim + qd * 32);
      kraw[2 * u] = p[0];
      kraw[2 * u + 1] = p[1];
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint4* p = reinterpret_cast<const uint4*>(vb + (dt * 16 + n) * kBlock + qd * 32);
      vraw[2 * dt] = p[0];
      vraw[2 * dt + 1] = p[1];
    }
  } else {
    const uint8_t* kb = kvd + kplane * (kBlock * kDim / 2);
    const uint8_t* vb = kvd + vplane * (kBlock * kDim / 2);
    const uint8_t* ks = kvs + kplane * (kBlock * kDim / 16);
    const uint8_t* vs = kvs + vplane * (kBlock * kDim / 16);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kappa = 32 * (n >> 2) + 8 * (u >> 1) + 4 * (u & 1) + (n & 3);
      kraw[u] = *reinterpret_cast<const uint4*>(kb + kappa * (kDim / 2) + qd * 16);
      ksc[u] = *reinterpret_cast<const uint16_t*>(ks + kappa * (kDim / 16) + qd * 2);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      vraw[dt] = *reinterpret_cast<const uint4*>(vb + (dt * 16 + n) * (kBlock / 2) + qd * 16);
      const uint4* sp = reinterpret_cast<const uint4*>(vs + dt * kBlock + qd * 32);
      vsc[2 * dt] = sp[0];
      vsc[2 * dt + 1] = sp[1];
    }
  }
  // ---- Q^T operand: head n of the group, dims qd*32 + 8c + e ----
  bf16x8 qop[4];
  if (n < a.hpg) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        q + ((size_t)si.row * a.H + (size_t)si.g * a.hpg + n) * kDim + qd * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[c] = __builtin_bit_cast(bf16x8, qp[c]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }

  // ---- S^T = K Q^T ----
  f32x4 sacc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    sacc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 kop;
      if constexpr (KV == kFP8) {
        const uint4 r = kraw[2 * u + (c >> 1)];
        kop = (c & 1) ? fp8x8_bf16(r.z, r.w) : fp8x8_bf16(r.x, r.y);
      } else {
        const uint32_t w = c == 0 ? kraw[u].x : c == 1 ? kraw[u].y : c == 2 ? kraw[u].z : kraw[u].w;
        const f32x2 sc = fp8x2_to_f32x2<false>(ksc[u]);
        kop = nvfp4x8_bf16(w, sc[c >> 1]);
      }
      sacc[u] = mfma_bf16(kop, qop[c], sacc[u]);
    }
  }

  // ---- softmax over the block's keys (head n lives in lanes n, n+16, n+32, n+48) ----
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 32 * qd + 8 * (u >> 1) + 4 * (u & 1) + i;
      const float t = key < si.nvalid ? sacc[u][i] * a.scale_log2 : -INFINITY;
      sacc[u][i] = t;
      mx = fmaxf(mx, t);
    }
  }
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  float lsum = 0.0f;
  f16x8 pop[4];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(sacc[u][i] - mx);
      lsum += p;
      pop[u >> 1][4 * (u & 1) + i] = (_Float16)p;
    }
  }
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);

  // ---- O = P V ----
  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f16x8 vop;
      if constexpr (KV == kFP8) {
        const uint4 r = vraw[2 * dt + (c >> 1)];
        vop = (c & 1) ? fp8x8_f16(r.z, r.w) : fp8x8_f16(r.x, r.y);
      } else {
        const uint32_t w = c == 0 ? vraw[dt].x : c == 1 ? vraw[dt].y : c == 2 ? vraw[dt].z : vraw[dt].w;
        const uint4 s = vsc[2 * dt + (c >> 1)];
        vop = (c & 1) ? nvfp4x8_f16(w, s.z, s.w) : nvfp4x8_f16(w, s.x, s.y);
      }
      oacc[dt] = mfma_f16(pop[c], vop, oacc[dt]);
    }
  }

  // ---- publish the partial ----
  const size_t pidx = (size_t)si.u * a.K + blockIdx.x;
  float* po = a.part_o + pidx * (kHeadsPad * 128);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) po[(4 * qd + i) * 128 + dt * 16 + n] = oacc[dt][i];
  }
  if (qd == 0) {
    float* pml = a.part_ml + pidx * (kHeadsPad * 2);
    pml[2 * n] = mx;
    pml[2 * n + 1] = lsum;
  }
  finish_split(a, si.u, si.count);
}

// ---------------------------------------------------------------------------
// fp32 cache (small exactness workloads): plain fp32 FMAs, same partials.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void attend_f32_kernel(const void* __restrict__ q,
                                                        const float* __restrict__ kvd,
                                                        int q_bf16, AttendArgs a) {
  __shared__ float qs[kHeadsPad][kDim];
  __shared__ float ps[kHeadsPad][kBlock];
  SplitInfo si;
  if (!split_info(a, si)) return;
  const int lane = threadIdx.x;
  if (si.pb < 0) {
    store_empty_partial(a, si);
    finish_split(a, si.u, si.count);
    return;
  }
  for (int i = lane; i < a.hpg * kDim; i += 64) {
    const size_t qi = ((size_t)si.row * a.H + (size_t)si.g * a.hpg) * kDim + i;
    qs[i / kDim][i % kDim] = q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(q)[qi])
                                    : reinterpret_cast<const float*>(q)[qi];
  }
  __syncthreads();
  const float* kb = kvd + (((size_t)si.pb * 2 + 0) * a.G + si.g) * (kBlock * kDim);
  const float* vb = kvd + (((size_t)si.pb * 2 + 1) * a.G + si.g) * (kBlock * kDim);
  float mh[kHeadsPad], lh[kHeadsPad];
  for (int h = 0; h < a.hpg; ++h) {
    float t[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int key = lane + 64 * half;
      const float4* kr = reinterpret_cast<const float4*>(kb + key * kDim);
      float acc = 0.0f;
      for (int d4 = 0; d4 < kDim / 4; ++d4) {
        const float4 k = kr[d4];
        acc = fmaf(qs[h][4 * d4], k.x, acc);
        acc = fmaf(qs[h][4 * d4 + 1], k.y, acc);
        acc = fmaf(qs[h][4 * d4 + 2], k.z, acc);
        acc = fmaf(qs[h][4 * d4 + 3], k.w, acc);
      }
      t[half] = key < si.nvalid ? acc * a.scale_log2 : -INFINITY;
    }
    const float m = wave_max(fmaxf(t[0], t[1]));
    const float p0 = exp2f(t[0] - m), p1 = exp2f(t[1] - m);
    ps[h][lane] = p0;
    ps[h][lane + 64] = p1;
    mh[h] = m;
    lh[h] = wave_sum(p0 + p1);
  }
  __syncthreads();
  const size_t pidx = (size_t)si.u * a.K + blockIdx.x;
  float* po = a.part_o + pidx * (kHeadsPad * 128);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int d = lane + 64 * half;
    const float4* vr = reinterpret_cast<const float4*>(vb + d * kBlock);
    for (int h = 0; h < a.hpg; ++h) {
      float acc = 0.0f;
      for (int k4 = 0; k4 < kBlock / 4; ++k4) {
        const float4 v = vr[k4];
        acc = fmaf(ps[h][4 * k4], v.x, acc);
        acc = fmaf(ps[h][4 * k4 + 1], v.y, acc);
        acc = fmaf(ps[h][4 * k4 + 2], v.z, acc);
        acc = fmaf(ps[h][4 * k4 + 3], v.w, acc);
      }
      po[h * 128 + d] = acc;
    }
  }
  if (lane == 0) {
    float* pml = a.part_ml + pidx * (kHeadsPad * 2);
    for (int h = 0; h < a.hpg; ++h) {
      pml[2 * h] = mh[h];
      pml[2 * h + 1] = lh[h];
    }
  }
  finish_split(a, si.u, si.count);
}

hipError_t launch_sparse_attend(const Shape& s, const void* q, const void* kv_data,
                                const void* kv_scales, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* q_pos,
                                const int32_t* topk, void* out, float* lse,
                                int32_t* counters, float* part_o, float* part_ml,
                                hipStream_t st) {
  AttendArgs a;
  a.bt = block_table;
  a.lens = seq_lens;
  a.qpos = q_pos;
  a.topk = topk;
  a.out = out;
  a.lse = lse;
  a.counters = counters;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.R = s.R;
  a.H = s.H;
  a.G = s.G;
  a.hpg = s.hpg;
  a.MB = s.MB;
  a.K = s.K;
  a.scale_log2 = s.sm_scale * s.k_scale * 1.4426950408889634f;
  a.v_scale = s.v_scale;
  a.out_f32 = s.out_dtype == kF32;
  dim3 grid(s.K, s.rows * s.G), block(64);
  if (s.kv_dtype == kFP8) {
    hipLaunchKernelGGL(attend_mfma_kernel<kFP8>, grid, block, 0, st, (const uint16_t*)q,
                       (const uint8_t*)kv_data, (const uint8_t*)nullptr, a);
  } else if (s.kv_dtype == kNVFP4) {
    hipLaunchKernelGGL(attend_mfma_kernel<kNVFP4>, grid, block, 0, st, (const uint16_t*)q,
                       (const uint8_t*)kv_data, (const uint8_t*)kv_scales, a);
  } else {
    hipLaunchKernelGGL(attend_f32_kernel, grid, block, 0, st, q, (const float*)kv_data,
                       (int)(s.q_dtype == kBF16), a);
  }
  return hipGetLastError();
}

}  // namespace msa
