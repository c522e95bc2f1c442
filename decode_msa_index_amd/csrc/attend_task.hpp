// attend_task.hpp -- exact GQA attention over selected KV blocks, as one
// task of a workgroup: shared by the attention kernels and the persistent
// decode kernel.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer" and Figure 1): every query head of a GQA group attends exactly the
// group's selected blocks, at most k*128 keys.  The attention itself is
// ordinary softmax attention, run split-K over the selected blocks (the API
// reference of MiniMaxM3SparseAttention._run_attention describes split-K
// attend kernels that read per-request metadata).
//
// A task is one (row, group) unit, or one of its S split-K shares: a
// workgroup of NW waves takes a contiguous share of the unit's selected
// blocks and wave w of it every NW-th entry of that share.  For a block of
// 128 keys and the group's (up to 16) heads a wave computes
//   S^T = K Q^T            v_mfma_f32_16x16x32_bf16  (K e4m3/e2m1 -> bf16 exact)
//   P   = exp2(S*scale - m) in fp32, rounded to f16 for the next product
//   O  += P V              v_mfma_f32_16x16x32_f16   (V e4m3/e2m1 -> f16 exact)
// with an online-softmax running state; the waves' states merge through LDS,
// and the S shares through device-scope stores and a last-arriver merge.
//
// Operand layout.  The contraction order inside an MFMA is free as long as
// both operands agree, so the key order of the S^T tiles is chosen to make
// every global load contiguous: tile u (0..7) row m holds key
//   kappa(u, m) = 32*(m/4) + 8*(u/2) + 4*(u%2) + m%4,
// which puts, for PV chunk c, keys 32*(l/16) + 8*c + 0..7 into lane l's
// eight A elements -- exactly the 8 consecutive bytes of a V^T row that the
// B operand needs (V is stored transposed, [d][t], for this).
#pragma once

#include "device.hpp"
#include "launch.hpp"
#include "select_wave.hpp"

namespace msa {

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
// Arguments shared by the kernels.
// ---------------------------------------------------------------------------
struct AttendArgs {
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* qpos;
  const int32_t* topk;    // selection input (attend only)
  const float* scores;    // pooled scores (select + attend, written by an earlier kernel)
  uint32_t* clear;        // SELECT: [units][MB] words the last reader zeroes (nullable)
  int32_t* topk_out;      // selection output (select + attend), may be null
  void* out;
  float* lse;
  int R, H, G, hpg, MB, K, P;
  float scale_log2;  // sm_scale * k_scale * log2(e)
  float v_scale;
  int out_f32;
};

__device__ __forceinline__ void store_out(const AttendArgs& a, int row, int h, int d, float v) {
  const size_t idx = ((size_t)row * a.H + h) * kDim + d;
  if (a.out_f32)
    reinterpret_cast<float*>(a.out)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(a.out)[idx] = f32_to_bf16(v);
}

// Dims d0 .. d0+7 of head h (d0 a multiple of 8): one 16-byte store (bf16)
// or two (f32).
__device__ __forceinline__ void store_out8(const AttendArgs& a, int row, int h, int d0,
                                           const float (&o)[8]) {
  const size_t idx = ((size_t)row * a.H + h) * kDim + d0;
  if (a.out_f32) {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + idx);
    p[0] = make_float4(o[0], o[1], o[2], o[3]);
    p[1] = make_float4(o[4], o[5], o[6], o[7]);
  } else {
    uint4 w;
    w.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
    w.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
    w.z = (uint32_t)f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
    w.w = (uint32_t)f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + idx) = w;
  }
}

// exp2(x - m) that is 0 when both are -inf (an empty partial)
__device__ __forceinline__ float rescale(float x, float m) {
  return x == -INFINITY ? 0.0f : exp2f(x - m);
}

// ---------------------------------------------------------------------------
// FP8 / NVFP4 cache, bf16 queries: MFMA tiles.
//
// Grid: (row, group) x S splits; a workgroup of NW waves takes a contiguous
// share of the row's selection entries and wave w of it takes every NW-th
// entry of that share.  With SELECT the workgroup first makes the group's
// selection itself from the pooled scores (wave 0, select_wave.hpp; every
// split recomputes it, which costs no extra latency) and split 0 also
// stores it.  For each block a wave computes S^T = K Q^T on MFMA, updates
// its running max / denominator (online softmax, fp32) and accumulates P V
// on MFMA into the rescaled running output.  The NW states of a workgroup
// merge pairwise through LDS.  With S = 1 the workgroup writes the
// normalised output; otherwise it publishes its state with coherent
// (device-scope) stores, and the last of the S workgroups to arrive -- a
// device-scope counter per (row, group) -- merges the S states and writes the
// output.  No cache write-back fence is needed: every value another
// workgroup reads is written and read with device-scope atomic accesses.
// Running state layout per lane l: max and denominator of head l%16; output
// rows (heads) 4*(l/16)+i, columns (dims) 16*dt + l%16.
// ---------------------------------------------------------------------------
struct Partials {
  float* o;          // [rows*G][S][16][128] unnormalised outputs
  float* ml;         // [rows*G][S][16][2]   running max (log2 domain) and denominator
  int32_t* counters; // [rows*G] arrivals, zero before the launch; reset by the merger
  int S;
};

// Host side: the argument blocks of an attention launch.
inline AttendArgs make_attend_args(const Shape& s, const int32_t* block_table,
                                   const int32_t* seq_lens, const int32_t* q_pos,
                                   const int32_t* topk, const float* scores, int32_t* topk_out,
                                   void* out, float* lse) {
  AttendArgs a{};
  a.bt = block_table;
  a.lens = seq_lens;
  a.qpos = q_pos;
  a.topk = topk;
  a.scores = scores;
  a.clear = nullptr;
  a.topk_out = topk_out;
  a.out = out;
  a.lse = lse;
  a.R = s.R;
  a.H = s.H;
  a.G = s.G;
  a.hpg = s.hpg;
  a.MB = s.MB;
  a.K = s.K;
  a.P = s.P;
  a.scale_log2 = s.sm_scale * s.k_scale * 1.4426950408889634f;
  a.v_scale = s.v_scale;
  a.out_f32 = s.out_dtype == kF32;
  return a;
}

// Split-K scratch inside the attention workspace (attend_workspace_bytes):
// [ml: units*S*16*2][o: units*S*16*128] floats, then [units] arrival counters.
inline Partials make_partials(const Shape& s, const AttendConfig& c, void* workspace) {
  const size_t units = (size_t)s.rows * s.G;
  Partials part;
  part.S = c.splits;
  part.ml = static_cast<float*>(workspace);
  part.o = part.ml + units * c.splits * kHeadsPad * 2;
  part.counters = reinterpret_cast<int32_t*>(part.o + units * c.splits * kHeadsPad * kDim);
  return part;
}

__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-scope (sc1) vector loads through a buffer resource over [base,
// base + bytes): data another workgroup of the same kernel wrote with
// device-scope stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
constexpr int kCoherentAux = 16;  // cache policy: sc1
__device__ __forceinline__ f32x4 coherent_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentAux));
}
__device__ __forceinline__ f32x2 coherent_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherentAux));
}

// Returns the unit's row of the scores to 0 once every reader is done with
// it, so that the workspace is left as the call found it.
__device__ __forceinline__ void clear_row(const AttendArgs& a, int u, int nw) {
  uint32_t* row = a.clear + (size_t)u * a.MB;
  for (int jj = threadIdx.x; jj < a.MB; jj += 64 * nw) row[jj] = 0u;
}

// One attention task: (row, group) unit u, split `split` of part.S, run by
// the calling workgroup of NW waves.  sel_lds: the dynamic LDS of a SELECT
// kernel.  Returns early (all threads of the workgroup together) where it
// has nothing more to do.
template <int KV, int NW, bool SELECT>
__device__ __forceinline__ void attend_task(const uint16_t* __restrict__ q,
                                            const uint8_t* __restrict__ kvd,
                                            const uint8_t* __restrict__ kvs, const AttendArgs& a,
                                            const Partials& part, int u, int split,
                                            uint32_t* sel_lds) {
  __shared__ float red_o[NW > 1 ? NW / 2 : 1][32][64];
  __shared__ float red_ml[NW > 1 ? NW / 2 : 1][2][16];
  __shared__ int32_t sel_w[SELECT ? NW : 1][32];  // SELECT: each wave's copy of the selection
  __shared__ int is_last;
  // sel_lds (SELECT): [256] scratch, [MB] keys, [MB] table row
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int row = u / a.G, g = u % a.G, b = row / a.R;
  const int pos = row_last_key(a.lens, a.qpos, row, b, a.MB);
  const int rb = pos < 0 ? -1 : pos / kBlock;
  const int count = min(a.K, rb + 1);  // 0 when the row sees no key
  const int per_wg = (count + part.S - 1) / part.S;
  const int e0 = split * per_wg, e1 = min(count, e0 + per_wg);
  const int n = lane & 15, qd = lane >> 4;

  // Q^T operand: head n of the group, dims qd*32 + 8c + e (zero past hpg);
  // loaded first so that its latency overlaps the selection
  bf16x8 qop[4];
  if (n < a.hpg) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        q + ((size_t)row * a.H + (size_t)g * a.hpg + n) * kDim + qd * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[c] = __builtin_bit_cast(bf16x8, qp[c]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }

  if constexpr (SELECT) {
    // every thread loads a share of the row's scores (as order keys) and of
    // its block-table entries, in one round that does not wait for the row
    // length, and keeps its best candidate; the workgroup then selects
    __shared__ GroupSelectLds<NW> gsl;
    uint32_t* keys = sel_lds + 256;
    int32_t* btl = reinterpret_cast<int32_t*>(keys + a.MB);
    const int32_t* brow = a.bt + (size_t)b * a.MB;
    uint64_t best = kNoCand;
    const float* srow = a.scores + (size_t)u * a.MB;
    for (int base = 0; base < a.MB; base += 8 * 64 * NW) {
      float v[8];
      int32_t e[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int jj = min(base + r * 64 * NW + (int)threadIdx.x, a.MB - 1);
        v[r] = srow[jj];
        e[r] = brow[jj];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int jj = base + r * 64 * NW + (int)threadIdx.x;
        if (jj < a.MB) {
          const uint32_t k = order_key(v[r]);
          keys[jj] = k;
          btl[jj] = e[r];
          if (jj < rb) best = max(best, pack_cand(k, jj));
        }
      }
    }
    group_select<NW>(keys, rb, a.K, best, gsl, sel_lds, sel_w[wave]);
    if (a.clear && part.S == 1) clear_row(a, u, NW);
    if (split == 0 && wave == 0 && a.topk_out && lane < a.K)
      a.topk_out[(size_t)u * a.K + lane] = sel_w[0][lane];
  }

  float M = -INFINITY, Lr = 0.0f;
  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // The wave's selection entries e0+wave, e0+wave+NW, ... and their physical
  // blocks, fetched by parallel lanes up front: lane i holds the i-th one.
  int my_j = -1, my_pb = -1;
  {
    const int sidx = e0 + wave + NW * lane;
    if (lane < 32 && sidx < e1) my_j = SELECT ? sel_w[wave][sidx] : a.topk[(size_t)u * a.K + sidx];
    if (my_j >= 0 && my_j <= rb)
      my_pb = SELECT ? reinterpret_cast<const int32_t*>(sel_lds + 256 + a.MB)[my_j]
                     : a.bt[(size_t)b * a.MB + my_j];
  }
  for (int it = 0; e0 + wave + NW * it < e1; ++it) {
    const int j = __shfl(my_j, it, 64);
    const int pb = __shfl(my_pb, it, 64);
    if (j < 0 || j > rb) continue;      // malformed selection entry: contributes nothing
    if (pb < 0 || pb >= a.P) continue;  // invalid table entry: contributes nothing
    const int nvalid = min(kBlock, pos - j * kBlock + 1);
    const size_t kplane = ((size_t)pb * 2 + 0) * a.G + g;
    const size_t vplane = ((size_t)pb * 2 + 1) * a.G + g;

    // ---- loads: K rows kappa(u, n), V^T rows dt*16+n; 32 dims / tokens each ----
    uint4 kraw[16], vraw[16];
    uint32_t ksc[8];
    uint4 vsc[16];
    if constexpr (KV == kFP8) {
      const uint8_t* kb = kvd + kplane * (kBlock * kDim);
      const uint8_t* vb = kvd + vplane * (kBlock * kDim);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int kappa = 32 * (n >> 2) + 8 * (t >> 1) + 4 * (t & 1) + (n & 3);
        const uint4* p = reinterpret_cast<const uint4*>(kb + kappa * kDim + qd * 32);
        kraw[2 * t] = p[0];
        kraw[2 * t + 1] = p[1];
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
      for (int t = 0; t < 8; ++t) {
        const int kappa = 32 * (n >> 2) + 8 * (t >> 1) + 4 * (t & 1) + (n & 3);
        kraw[t] = *reinterpret_cast<const uint4*>(kb + kappa * (kDim / 2) + qd * 16);
        ksc[t] = *reinterpret_cast<const uint16_t*>(ks + kappa * (kDim / 16) + qd * 2);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        vraw[dt] = *reinterpret_cast<const uint4*>(vb + (dt * 16 + n) * (kBlock / 2) + qd * 16);
        const uint4* sp = reinterpret_cast<const uint4*>(vs + dt * kBlock + qd * 32);
        vsc[2 * dt] = sp[0];
        vsc[2 * dt + 1] = sp[1];
      }
    }

    // ---- S^T = K Q^T ----
    f32x4 sacc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      sacc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x8 kop;
        if constexpr (KV == kFP8) {
          const uint4 r = kraw[2 * t + (c >> 1)];
          kop = (c & 1) ? fp8x8_bf16(r.z, r.w) : fp8x8_bf16(r.x, r.y);
        } else {
          const uint32_t w = c == 0 ? kraw[t].x : c == 1 ? kraw[t].y : c == 2 ? kraw[t].z : kraw[t].w;
          const f32x2 sc = fp8x2_to_f32x2<false>(ksc[t]);
          kop = nvfp4x8_bf16(w, sc[c >> 1]);
        }
        sacc[t] = mfma_bf16(kop, qop[c], sacc[t]);
      }
    }

    // ---- online softmax update (head n lives in lanes n, n+16, n+32, n+48) ----
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 32 * qd + 8 * (t >> 1) + 4 * (t & 1) + i;
        const float v = key < nvalid ? sacc[t][i] * a.scale_log2 : -INFINITY;
        sacc[t][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float Mn = fmaxf(M, mx);
    const float alpha = rescale(M, Mn);
    float lsum = 0.0f;
    f16x8 pop[4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sacc[t][i] - Mn);
        lsum += p;
        pop[t >> 1][4 * (t & 1) + i] = (_Float16)p;
      }
    }
    lsum += shfl_xor(lsum, 16);
    lsum += shfl_xor(lsum, 32);
    Lr = Lr * alpha + lsum;
    M = Mn;
    float alpha_o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) alpha_o[i] = __shfl(alpha, 4 * qd + i, 64);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha_o[i];
    }

    // ---- O += P V ----
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f16x8 vop;
        if constexpr (KV == kFP8) {
          const uint4 r = vraw[2 * dt + (c >> 1)];
          vop = (c & 1) ? fp8x8_f16(r.z, r.w) : fp8x8_f16(r.x, r.y);
        } else {
          const uint32_t w = c == 0 ? vraw[dt].x : c == 1 ? vraw[dt].y : c == 2 ? vraw[dt].z : vraw[dt].w;
          const uint4 sv = vsc[2 * dt + (c >> 1)];
          vop = (c & 1) ? nvfp4x8_f16(w, sv.z, sv.w) : nvfp4x8_f16(w, sv.x, sv.y);
        }
        oacc[dt] = mfma_f16(pop[c], vop, oacc[dt]);
      }
    }
  }

  // ---- merge the waves' states pairwise through LDS ----
#pragma unroll
  for (int half = NW / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
      const int slot = wave - half;
      if (qd == 0) {
        red_ml[slot][0][n] = M;
        red_ml[slot][1][n] = Lr;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[slot][dt * 4 + i][lane] = oacc[dt][i];
      }
    }
    __syncthreads();
    if (wave < half) {
      const float Mb = red_ml[wave][0][n], Lb = red_ml[wave][1][n];
      const float Mn = fmaxf(M, Mb);
      const float fa = rescale(M, Mn), fb = rescale(Mb, Mn);
      Lr = Lr * fa + Lb * fb;
      M = Mn;
      float fa_o[4], fb_o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa_o[i] = __shfl(fa, 4 * qd + i, 64);
        fb_o[i] = __shfl(fb, 4 * qd + i, 64);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[dt][i] = oacc[dt][i] * fa_o[i] + red_o[wave][dt * 4 + i][lane] * fb_o[i];
      }
    }
    __syncthreads();
  }

  if (part.S == 1) {
    if (wave != 0) return;
    float inv_o[4];
    const float inv = Lr > 0.0f ? a.v_scale / Lr : 0.0f;  // no visible key: zeros
#pragma unroll
    for (int i = 0; i < 4; ++i) inv_o[i] = __shfl(inv, 4 * qd + i, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * qd + i;
      if (h < a.hpg) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          store_out(a, row, g * a.hpg + h, dt * 16 + n, oacc[dt][i] * inv_o[i]);
      }
    }
    if (a.lse && qd == 0 && n < a.hpg)
      a.lse[(size_t)row * a.H + (size_t)g * a.hpg + n] =
          Lr > 0.0f ? (M + log2f(Lr)) * 0.69314718055994531f : -INFINITY;
    return;
  }

  // ---- split-K across workgroups: publish, count arrivals, last one merges ----
  if (wave == 0) {
    const size_t pidx = (size_t)u * part.S + split;
    float* po = part.o + pidx * (kHeadsPad * kDim);
    // lane-major: value (dt, i) of lane l at (4 dt + i) * 64 + l, so each
    // store instruction writes 256 contiguous bytes
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) coherent_store(po + (4 * dt + i) * 64 + lane, oacc[dt][i]);
    }
    if (qd == 0) {
      coherent_store(part.ml + pidx * (kHeadsPad * 2) + 2 * n, M);
      coherent_store(part.ml + pidx * (kHeadsPad * 2) + 2 * n + 1, Lr);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    int prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(part.counters + u, 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, 64);
    if (lane == 0) is_last = prev == part.S - 1;
  }
  __syncthreads();
  if (!is_last) return;
  // merge: thread t takes head h = t/16 and dims d0 = 8*(t%16) .. +8
  // (looping when NW < 4).  Head h = 4*qd + i, dim 16*dt + n sits at
  // (4 dt + i) * 64 + 16 qd + n in a partial, so the 8 dims are 32
  // contiguous bytes: two 16-byte device-scope loads per partial, all issued
  // before any is used.  Each thread then zeroes what it read (and the
  // padded heads' entries), leaving the workspace as the call found it.
  const size_t ubase = (size_t)u * part.S;
  const __amdgpu_buffer_rsrc_t ro =
      coherent_rsrc(part.o + ubase * (kHeadsPad * kDim), part.S * kHeadsPad * kDim * 4);
  const __amdgpu_buffer_rsrc_t rm =
      coherent_rsrc(part.ml + ubase * (kHeadsPad * 2), part.S * kHeadsPad * 2 * 4);
  for (int t = threadIdx.x; t < kHeadsPad * 16; t += 64 * NW) {
    const int h = t >> 4, d0 = (t & 15) * 8;
    const int off = (4 * (d0 >> 4) + (h & 3)) * 64 + 16 * (h >> 2) + (d0 & 15);  // floats
    float* po = part.o + ubase * (kHeadsPad * kDim) + off;
    float* ml = part.ml + ubase * (kHeadsPad * 2) + 2 * h;
    if (h < a.hpg) {
      float pm[kMaxSplits], pl[kMaxSplits], pv[kMaxSplits][8];
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp) {
        if (sp < part.S) {
          const f32x2 m2 = coherent_load8(rm, (uint32_t)((sp * kHeadsPad + h) * 2 * 4));
          pm[sp] = m2[0];
          pl[sp] = m2[1];
          const uint32_t ob = (uint32_t)((sp * kHeadsPad * kDim + off) * 4);
          const f32x4 v0 = coherent_load16(ro, ob), v1 = coherent_load16(ro, ob + 16);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            pv[sp][k] = v0[k];
            pv[sp][4 + k] = v1[k];
          }
        }
      }
      float Mx = -INFINITY;
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp)
        if (sp < part.S) Mx = fmaxf(Mx, pm[sp]);
      float L = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp) {
        if (sp < part.S) {
          const float f = rescale(pm[sp], Mx);
          L += f * pl[sp];
#pragma unroll
          for (int k = 0; k < 8; ++k) o[k] += f * pv[sp][k];
        }
      }
      const float inv = L > 0.0f ? a.v_scale / L : 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= inv;
      store_out8(a, row, g * a.hpg + h, d0, o);
      if (a.lse && (t & 15) == 0)
        a.lse[(size_t)row * a.H + (size_t)g * a.hpg + h] =
            L > 0.0f ? (Mx + log2f(L)) * 0.69314718055994531f : -INFINITY;
    }
    for (int sp = 0; sp < part.S; ++sp) {
      float4* z = reinterpret_cast<float4*>(po + (size_t)sp * (kHeadsPad * kDim));
      z[0] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      z[1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if ((t & 15) == 0) *reinterpret_cast<float2*>(ml + (size_t)sp * (kHeadsPad * 2)) = make_float2(0.0f, 0.0f);
    }
  }
  if (SELECT && a.clear) clear_row(a, u, NW);
  if (threadIdx.x == 0)
    __hip_atomic_store(part.counters + u, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace msa
