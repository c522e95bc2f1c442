// attend_task.hpp -- exact GQA attention over selected KV blocks, as one
// task of a workgroup of the attention kernels (sparse_attend.hip).
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
// and the S shares through coherent stores that the unit's last share polls
// for and merges.
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
  int32_t* topk_out;      // selection output (select + attend), may be null
  void* out;
  float* lse;
  int R, H, G, hpg, MB, K, P;
  int init, local;   // forced blocks (select + attend): first `init`, last `local` (>= 1)
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

// 2^x on the hardware exp2 instruction alone, without the library's scaling
// for results below 2^-126 (those may come out as 0 rather than subnormal).
// Used for the attention weights 2^(s - max): a weight that small rounds to
// 0 in f16 for the P V product either way, and cannot change the fp32 row
// sum, which already holds the weight 1 of the row's maximum.
__device__ __forceinline__ float exp2_weight(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(x - m) that is 0 when both are -inf (an empty partial)
__device__ __forceinline__ float rescale(float x, float m) {
  return x == -INFINITY ? 0.0f : exp2f(x - m);
}

// ---------------------------------------------------------------------------
// FP8 / NVFP4 cache, bf16 queries: MFMA tiles.
//
// Grid: (row, group) x S splits; a workgroup of NW waves takes a contiguous
// share of the row's selection entries (in ascending block order, so a
// selection made here and a given one are attended alike) and wave w of it
// takes every NW-th entry of that share.  With SELECT the workgroup first
// makes the group's selection itself from the pooled scores
// (select_wave.hpp; every split recomputes it, which costs no extra latency)
// and split 0 also stores it.
// For each block a wave computes S^T = K Q^T on MFMA, updates its running
// max / denominator (online softmax, fp32) and accumulates P V on MFMA into
// the rescaled running output.  The NW states then meet in LDS, where wave w
// combines a 1/NW slice of the head dims for all heads.  With S = 1 each
// wave normalises and stores its slice.  With S > 1, splits 0 .. S-2 store
// their combined states with device-scope stores and leave; split S-1 (the
// highest workgroup id of the unit, so the other splits are already
// dispatched when it runs) polls for those states -- each word is encoded so
// that zero means "not yet written" -- merges them into its own, stores the
// output and then returns what it read to zero.  The launch makes sure all
// workgroups of the grid can be resident at once.
// Running state layout per lane l: max and denominator of head l%16; output
// rows (heads) 4*(l/16)+i, columns (dims) 16*dt + l%16.
// ---------------------------------------------------------------------------
struct Partials {
  float* o;          // [rows*G][S][8 dim tiles][64 lanes][4]: unnormalised outputs, lane-major
  float* ml;         // [rows*G][S][16 heads][2]: running max (log2 domain) and denominator
  uint32_t* status;  // the workspace's status word: non-zero once a merge has given up
  int S;
  int spin_limit;    // polls of one batch before a merger gives up (< 0: at once)
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
  a.init = s.init;
  a.local = s.local;
  a.scale_log2 = s.sm_scale * s.k_scale * 1.4426950408889634f;
  a.v_scale = s.v_scale;
  a.out_f32 = s.out_dtype == kF32;
  return a;
}

// Split-K scratch inside the attention workspace (attend_workspace_bytes):
// [ml: units*S*16*2][o: units*S*16*128] floats.  Zero before a launch, and
// zero again after it (the merging workgroup clears what it read).
inline Partials make_partials(const Shape& s, const AttendConfig& c, void* workspace,
                              uint32_t* status, int spin_limit) {
  const size_t units = (size_t)s.rows * s.G;
  Partials part;
  part.S = c.splits;
  part.ml = static_cast<float*>(workspace);
  part.o = part.ml + units * c.splits * kHeadsPad * 2;
  part.status = status;
  part.spin_limit = spin_limit;
  return part;
}

// Device-scope (sc1) 16-byte accesses through a buffer resource over [base,
// base + bytes): stores that write through to the device's coherence point
// and loads that read from it, for data other workgroups of the same kernel
// exchange while it runs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
constexpr int kCoherentAux = 16;  // cache policy: sc1
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 coherent_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentAux));
}
__device__ __forceinline__ void coherent_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kCoherentAux);
}

// Partial states travel with every 32-bit word stored as bits ^ kPartialXor.
// kPartialXor is itself a NaN pattern, and NaNs are stored as the canonical
// quiet NaN first, so an encoded word is never 0: a reader polling
// zero-filled memory knows each word it sees non-zero is complete -- no
// flag, fence or counter is needed.
constexpr uint32_t kPartialXor = 0x7FFFFFFFu;
constexpr uint32_t kQuietNaN = 0x7FC00000u;
__device__ __forceinline__ f32x4 encode_partial(f32x4 v) {
  u32x4_t w = __builtin_bit_cast(u32x4_t, v);
  w.x = (v[0] != v[0] ? kQuietNaN : w.x) ^ kPartialXor;
  w.y = (v[1] != v[1] ? kQuietNaN : w.y) ^ kPartialXor;
  w.z = (v[2] != v[2] ? kQuietNaN : w.z) ^ kPartialXor;
  w.w = (v[3] != v[3] ? kQuietNaN : w.w) ^ kPartialXor;
  return __builtin_bit_cast(f32x4, w);
}
__device__ __forceinline__ f32x4 decode_partial(f32x4 v) {
  u32x4_t w = __builtin_bit_cast(u32x4_t, v);
  w ^= kPartialXor;
  return __builtin_bit_cast(f32x4, w);
}
__device__ __forceinline__ bool all_landed(f32x4 v) {
  const u32x4_t w = __builtin_bit_cast(u32x4_t, v);
  return w.x != 0u && w.y != 0u && w.z != 0u && w.w != 0u;
}
// Polls of one batch of partials before the merger gives up (each poll is a
// device-memory round trip, about a microsecond): the default of
// Partials::spin_limit.
constexpr int kSpinLimit = 1 << 20;

// The state arithmetic below writes every multiply-add as an explicit fmaf:
// a sum of two products left to the compiler may be fused either way, and
// the kernels that attend a unit (given selection, selection made in-kernel)
// must round it alike.

// Where a task's selection comes from.
enum SelMode {
  kSelGiven = 0,  // topk_idx, an input
  kSelScores = 1  // made here from pooled scores an earlier kernel wrote
};

// One attention task: (row, group) unit u, split `split` of part.S, run by
// the calling workgroup of NW waves.  sel_lds: the dynamic LDS of a
// selecting kernel.  Returns early (all threads of the workgroup together)
// where it has nothing more to do.
template <int KV, int NW, int SEL>
__device__ __forceinline__ void attend_task(const uint16_t* __restrict__ q,
                                            const uint8_t* __restrict__ kvd,
                                            const uint8_t* __restrict__ kvs, const AttendArgs& a,
                                            const Partials& part, int u, int split,
                                            uint32_t* sel_lds) {
  constexpr bool SELECT = SEL != kSelGiven;
  __shared__ int32_t sel_w[SELECT ? NW : 1][32];  // SELECT: each wave's copy of the selection
  __shared__ uint4 vsl[KV == kNVFP4 ? NW : 1][64];  // NVFP4: each wave's block of V scales
  // sel_lds (SELECT): [256] scratch, [MB] keys, then (kSelScores) [MB] table row
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int row = u / a.G, g = u % a.G, b = row / a.R;
  const int pos = row_last_key(a.lens, a.qpos, row, b, a.MB);
  const int rb = pos < 0 ? -1 : pos / kBlock;
  const int count = min(a.K, rb + 1);  // 0 when the row sees no key
  const int per_wg = (count + part.S - 1) / part.S;
  const int e0 = split * per_wg, e1 = min(count, e0 + per_wg);
  const int n = lane & 15, qd = lane >> 4;
  // the merging split reads the workspace's status word early: a workspace
  // a merge gave up on holds partial words that may still land late, so its
  // partials are not trusted again until the caller clears it
  const uint32_t poisoned = (part.S > 1 && split == part.S - 1) ? *part.status : 0u;

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

  int sorted_sel = -1;  // SELECT: lane l's entry of the ascending selection
  if constexpr (SEL == kSelScores) {
    // every thread loads a share of the row's scores (as order keys) and of
    // its block-table entries, in one round that does not wait for the row
    // length, and keeps its largest key; the workgroup then selects
    __shared__ GroupSelectLds<NW> gsl;
    uint32_t* keys = sel_lds + 256;
    int32_t* btl = reinterpret_cast<int32_t*>(keys + a.MB);
    const int32_t* brow = a.bt + (size_t)b * a.MB;
    uint32_t tmax = 0u;
    const int c0 = a.init, c1 = rb + 1 - a.local;  // the free candidates
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
          if (jj >= c0 && jj < c1) tmax = max(tmax, k);
        }
      }
    }
    group_select<NW>(keys, rb, a.K, a.init, a.local, tmax, gsl, sel_lds, sel_w[wave]);
    // the selection in ascending order, as msa_block_topk stores it: the
    // blocks are then attended in the same order as from a given selection
    sorted_sel = sort_selection(lane < a.K ? sel_w[wave][lane] : -1, a.K);
    if (split == 0 && wave == 0 && a.topk_out && lane < a.K)
      a.topk_out[(size_t)u * a.K + lane] = sorted_sel;
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
    const int sel_e = SELECT ? __shfl(sorted_sel, min(sidx, 63), 64) : -1;
    if (lane < 32 && sidx < e1) my_j = SELECT ? sel_e : a.topk[(size_t)u * a.K + sidx];
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
    uint4 vsc;  // NVFP4: 16 bytes of the block's V scales (staged in LDS for the P V step)
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
      for (int dt = 0; dt < 8; ++dt)
        vraw[dt] = *reinterpret_cast<const uint4*>(vb + (dt * 16 + n) * (kBlock / 2) + qd * 16);
      // the block's 1 KB of V scales ([d/16][t]), 16 bytes per lane: every
      // lane needs 8 of them per 8-key chunk, and 16 lanes the same ones
      vsc = reinterpret_cast<const uint4*>(vs)[lane];
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
    // (Measured slower: the block maximum on raw logits with one fma per
    // weight, 1.5 us per 32 x 32K decode step.)
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
        const float p = exp2_weight(sacc[t][i] - Mn);
        lsum += p;
        pop[t >> 1][4 * (t & 1) + i] = (_Float16)p;
      }
    }
    lsum += shfl_xor(lsum, 16);
    lsum += shfl_xor(lsum, 32);
    Lr = fmaf(Lr, alpha, lsum);
    M = Mn;
    {
      float alpha_o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) alpha_o[i] = __shfl(alpha, 4 * qd + i, 64);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= alpha_o[i];
      }
    }

    // ---- O += P V ----
    if constexpr (KV == kNVFP4) {  // the V scales through the wave's LDS slice
      wave_lds_sync();  // the previous block's reads are done
      vsl[wave][lane] = vsc;
      wave_lds_sync();
    }
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
          // scales of keys 32 qd + 8 c .. +7 in dim row dt (one per 16 dims)
          const uint2 sv = *reinterpret_cast<const uint2*>(
              reinterpret_cast<const uint8_t*>(vsl[wave]) + dt * kBlock + 32 * qd + 8 * c);
          vop = nvfp4x8_f16(w, sv.x, sv.y);
        }
        oacc[dt] = mfma_f16(pop[c], vop, oacc[dt]);
      }
    }
  }

  // ---- combine the NW waves' states: each wave stores its state in LDS,
  // then wave w combines dims [16 w DTW, +16 DTW) of all heads ----
  constexpr int DTW = 8 / NW;  // 16-dim tiles per wave after the combine
  f32x4 co[DTW];               // combined output: heads 4qd+i, dims 16 d + n
  float cm[4], cl[4];          // combined max (log2 domain) and denominator of heads 4qd+i
  if constexpr (NW == 1) {
#pragma unroll
    for (int d = 0; d < DTW; ++d) co[d] = oacc[d];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cm[i] = __shfl(M, 4 * qd + i, 64);
      cl[i] = __shfl(Lr, 4 * qd + i, 64);
    }
  } else {
    __shared__ f32x4 st_o[NW][8][64];
    __shared__ f32x2 st_ml[NW][kHeadsPad];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st_o[wave][dt][lane] = oacc[dt];
    if (qd == 0) st_ml[wave][n] = f32x2{M, Lr};
    __syncthreads();
    float f[NW][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cm[i] = -INFINITY;
    float l[NW][4];
#pragma unroll
    for (int v = 0; v < NW; ++v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 ml = st_ml[v][4 * qd + i];
        f[v][i] = ml[0];
        l[v][i] = ml[1];
        cm[i] = fmaxf(cm[i], ml[0]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) cl[i] = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[v][i] = rescale(f[v][i], cm[i]);
        cl[i] = fmaf(f[v][i], l[v][i], cl[i]);
      }
    }
#pragma unroll
    for (int d = 0; d < DTW; ++d) {
      co[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const f32x4 x = st_o[v][wave * DTW + d][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) co[d][i] = fmaf(f[v][i], x[i], co[d][i]);
      }
    }
  }
  const int dt0 = wave * DTW;  // first 16-dim tile this wave holds

  // ---- split-K across workgroups: splits 0 .. S-2 publish their states;
  // split S-1 polls for them and merges ----
  if (part.S > 1 && split < part.S - 1) {
    // every word is stored as bits ^ kPartialXor, which is never 0 (see
    // kPartialXor), so a reader sees 0 until the store has landed
    const size_t pidx = (size_t)u * part.S + split;
    const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(part.o + pidx * (kHeadsPad * kDim),
                                                    kHeadsPad * kDim * 4);
#pragma unroll
    for (int d = 0; d < DTW; ++d)
      coherent_store16(ro, (uint32_t)(((dt0 + d) * 64 + lane) * 16), encode_partial(co[d]));
    if (wave == 0 && n == 0) {  // lanes 0, 16, 32, 48: heads 4qd .. 4qd+3
      const __amdgpu_buffer_rsrc_t rm = coherent_rsrc(part.ml + pidx * (kHeadsPad * 2),
                                                      kHeadsPad * 2 * 4);
      coherent_store16(rm, (uint32_t)(qd * 32),
                       encode_partial(f32x4{cm[0], cl[0], cm[1], cl[1]}));
      coherent_store16(rm, (uint32_t)(qd * 32 + 16),
                       encode_partial(f32x4{cm[2], cl[2], cm[3], cl[3]}));
    }
    return;
  }
  bool timed_out = poisoned != 0u || (part.S > 1 && part.spin_limit < 0);
  if (part.S > 1) {
    // merge the other splits' partials, a batch at a time, into (co, cm, cl)
    constexpr int CH = 128 / (4 * DTW + 8);  // partials whose words a batch holds
    const size_t ubase = (size_t)u * part.S;
    for (int sp0 = 0; sp0 < part.S - 1 && !timed_out; sp0 += CH) {
      f32x4 po[CH][DTW], pm[CH][2];
      for (int tries = 0;; ++tries) {
        // the loads below must be issued again on every pass: without this
        // barrier the compiler may hoist them out of the loop
        asm volatile("" ::: "memory");
        bool ok = true;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int sp = sp0 + c;
          if (sp < part.S - 1) {
            const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(
                part.o + (ubase + sp) * (kHeadsPad * kDim), kHeadsPad * kDim * 4);
            const __amdgpu_buffer_rsrc_t rm = coherent_rsrc(
                part.ml + (ubase + sp) * (kHeadsPad * 2), kHeadsPad * 2 * 4);
#pragma unroll
            for (int d = 0; d < DTW; ++d)
              po[c][d] = coherent_load16(ro, (uint32_t)(((dt0 + d) * 64 + lane) * 16));
            pm[c][0] = coherent_load16(rm, (uint32_t)(qd * 32));
            pm[c][1] = coherent_load16(rm, (uint32_t)(qd * 32 + 16));
#pragma unroll
            for (int d = 0; d < DTW; ++d) ok = ok && all_landed(po[c][d]);
            ok = ok && all_landed(pm[c][0]) && all_landed(pm[c][1]);
          }
        }
        if (__ballot(!ok) == 0) break;
        if (tries >= part.spin_limit) {  // never expected: the output becomes NaN
          timed_out = true;
          break;
        }
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (sp0 + c < part.S - 1) {
          const f32x4 m0 = decode_partial(pm[c][0]), m1 = decode_partial(pm[c][1]);
          const float sm[4] = {m0[0], m0[2], m1[0], m1[2]};
          const float sl[4] = {m0[1], m0[3], m1[1], m1[3]};
          float fa[4], fb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float mx = fmaxf(cm[i], sm[i]);
            fa[i] = rescale(cm[i], mx);
            fb[i] = rescale(sm[i], mx);
            cm[i] = mx;
            cl[i] = fmaf(sl[i], fb[i], cl[i] * fa[i]);
          }
#pragma unroll
          for (int d = 0; d < DTW; ++d) {
            const f32x4 x = decode_partial(po[c][d]);
#pragma unroll
            for (int i = 0; i < 4; ++i) co[d][i] = fmaf(x[i], fb[i], co[d][i] * fa[i]);
          }
        }
      }
    }
    // one verdict for the workgroup (each wave polled its own words), and
    // every wave is past its polls before any of them clears a shared word
    timed_out = __syncthreads_or(timed_out ? 1 : 0) != 0;
  }

  // ---- normalise and store (heads 4qd+i, dims 16 (dt0 + d) + n) ----
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    inv[i] = timed_out ? __builtin_nanf("") : (cl[i] > 0.0f ? a.v_scale / cl[i] : 0.0f);
  if constexpr (NW <= 4) {
    // 8 consecutive dims of one head per lane: the wave's values meet in
    // LDS -- each wave its own dims, so a wave-level sync orders the
    // accesses -- and leave as 16-byte stores.  (Eight-wave workgroups keep
    // the element stores: the extra registers cost them more than they save.)
    __shared__ float ob[kHeadsPad][kDim + 4];  // +4: rows start on different banks
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int d = 0; d < DTW; ++d) ob[4 * qd + i][(dt0 + d) * 16 + n] = co[d][i] * inv[i];
    }
    wave_lds_sync();
    constexpr int CPH = 2 * DTW;  // 8-dim chunks of a head in the wave's dims
#pragma unroll
    for (int c0 = 0; c0 < kHeadsPad * CPH; c0 += 64) {
      const int c = c0 + lane, h = c / CPH, d0 = dt0 * 16 + (c % CPH) * 8;
      if (c < kHeadsPad * CPH && h < a.hpg) {
        const float4 lo = *reinterpret_cast<const float4*>(&ob[h][d0]);
        const float4 hi = *reinterpret_cast<const float4*>(&ob[h][d0 + 4]);
        const float o[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        store_out8(a, row, g * a.hpg + h, d0, o);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * qd + i;
      if (h < a.hpg) {
#pragma unroll
        for (int d = 0; d < DTW; ++d)
          store_out(a, row, g * a.hpg + h, (dt0 + d) * 16 + n, co[d][i] * inv[i]);
      }
    }
  }
  if (a.lse && wave == 0 && n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * qd + i;
      if (h < a.hpg)
        a.lse[(size_t)row * a.H + (size_t)g * a.hpg + h] =
            timed_out ? __builtin_nanf("")
                      : (cl[i] > 0.0f ? (cm[i] + log2f(cl[i])) * 0.69314718055994531f : -INFINITY);
    }
  }

  // ---- the merger, after its output: return the partials it read to zero,
  // so the workspace is left as found (all waves are past their polls: the
  // barrier after the merge).  After a timeout nothing is cleared (a late
  // partial could land after the clearing); the status word marks the
  // workspace instead, for the host to read and to clear. ----
  if (part.S > 1) {
    const size_t ubase = (size_t)u * part.S;
    if (timed_out) {
      if (threadIdx.x == 0) *part.status = 1u;
      return;
    }
#pragma unroll 1
    for (int sp = 0; sp < part.S - 1; ++sp) {
      f32x4* zo = reinterpret_cast<f32x4*>(part.o + (ubase + sp) * (kHeadsPad * kDim));
#pragma unroll
      for (int d = 0; d < DTW; ++d) zo[(dt0 + d) * 64 + lane] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (wave == 0 && n == 0) {
        f32x4* zm = reinterpret_cast<f32x4*>(part.ml + (ubase + sp) * (kHeadsPad * 2));
        zm[2 * qd] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        zm[2 * qd + 1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  }
}

}  // namespace msa
