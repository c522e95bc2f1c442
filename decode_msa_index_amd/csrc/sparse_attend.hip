// sparse_attend.hip -- the attention kernels and their launch shapes.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer" and Figure 1): every query head of a GQA group attends exactly the
// group's selected blocks, at most k*128 keys; the attention itself is
// ordinary softmax attention, here split-K over the selected blocks (the API
// reference of MiniMaxM3SparseAttention._run_attention describes split-K
// attend kernels that read per-request metadata).
//
// attend_mfma_kernel runs one attend_task (attend_task.hpp) per workgroup:
// grid = (row, group) units x S splits.  Its SELECT form first makes the
// group's block selection from the pooled scores (msa_decode's second
// kernel).  attend_f32_kernel is the plain fp32 path for fp32 caches.
#include "attend_task.hpp"
#include "device.hpp"
#include "launch.hpp"

#include <atomic>
#include <mutex>
#include <vector>

namespace msa {

// At most 256 registers per lane (VGPRs and AGPRs together), so that every
// form keeps 2 waves per SIMD: the one-wave form, used for grids of many
// units, came out a few registers past that (1 wave per SIMD) on its own.
template <int KV, int NW, bool SELECT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void attend_mfma_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kvd,
    const uint8_t* __restrict__ kvs, AttendArgs a, Partials part) {
  extern __shared__ uint32_t sel_lds[];
  attend_task<KV, NW, SELECT ? kSelScores : kSelGiven>(q, kvd, kvs, a, part, blockIdx.x / part.S,
                                                      blockIdx.x % part.S, sel_lds);
}

__global__ void zero_fill_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Clears bytes (a multiple of 4) at p with a fill kernel (no memset node, so
// the call can sit inside a captured graph).
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  if (n > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     static_cast<int32_t*>(p), (int)n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 cache (small exactness workloads): one wave per (row, group) walks
// the selected blocks with plain fp32 FMAs and an online softmax.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void attend_f32_kernel(const void* __restrict__ q,
                                                        const float* __restrict__ kvd,
                                                        int q_bf16, AttendArgs a) {
  __shared__ float qs[kHeadsPad][kDim];
  __shared__ float ps[kHeadsPad][kBlock];
  __shared__ float alpha_s[kHeadsPad];
  const int lane = threadIdx.x;
  const int u = blockIdx.x, row = u / a.G, g = u % a.G, b = row / a.R;
  const int pos = row_last_key(a.lens, a.qpos, row, b, a.MB);
  const int rb = pos < 0 ? -1 : pos / kBlock;
  const int count = min(a.K, rb + 1);  // 0 when the row sees no key
  for (int i = lane; i < a.hpg * kDim; i += 64) {
    const size_t qi = ((size_t)row * a.H + (size_t)g * a.hpg) * kDim + i;
    qs[i / kDim][i % kDim] = q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(q)[qi])
                                    : reinterpret_cast<const float*>(q)[qi];
  }
  float M[kHeadsPad], Lr[kHeadsPad], o0[kHeadsPad], o1[kHeadsPad];
  for (int h = 0; h < kHeadsPad; ++h) {
    M[h] = -INFINITY;
    Lr[h] = 0.0f;
    o0[h] = o1[h] = 0.0f;
  }
  __syncthreads();
  for (int sidx = 0; sidx < count; ++sidx) {
    const int j = a.topk[(size_t)u * a.K + sidx];
    if (j < 0 || j > rb) continue;
    const int pb = a.bt[(size_t)b * a.MB + j];
    if (pb < 0 || pb >= a.P) continue;  // invalid table entry: contributes nothing
    const int nvalid = min(kBlock, pos - j * kBlock + 1);
    const float* kb = kvd + (((size_t)pb * 2 + 0) * a.G + g) * (kBlock * kDim);
    const float* vb = kvd + (((size_t)pb * 2 + 1) * a.G + g) * (kBlock * kDim);
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
        t[half] = key < nvalid ? acc * a.scale_log2 : -INFINITY;
      }
      const float mx = wave_max(fmaxf(t[0], t[1]));
      const float Mn = fmaxf(M[h], mx);
      const float al = rescale(M[h], Mn);
      const float p0 = exp2f(t[0] - Mn), p1 = exp2f(t[1] - Mn);
      ps[h][lane] = p0;
      ps[h][lane + 64] = p1;
      Lr[h] = Lr[h] * al + wave_sum(p0 + p1);
      M[h] = Mn;
      if (lane == 0) alpha_s[h] = al;
    }
    __syncthreads();
    for (int h = 0; h < a.hpg; ++h) {
      const float al = alpha_s[h];
      float acc0 = 0.0f, acc1 = 0.0f;
      const float4* v0 = reinterpret_cast<const float4*>(vb + lane * kBlock);
      const float4* v1 = reinterpret_cast<const float4*>(vb + (lane + 64) * kBlock);
      for (int k4 = 0; k4 < kBlock / 4; ++k4) {
        const float4 x = v0[k4], y = v1[k4];
        acc0 = fmaf(ps[h][4 * k4], x.x, acc0);
        acc0 = fmaf(ps[h][4 * k4 + 1], x.y, acc0);
        acc0 = fmaf(ps[h][4 * k4 + 2], x.z, acc0);
        acc0 = fmaf(ps[h][4 * k4 + 3], x.w, acc0);
        acc1 = fmaf(ps[h][4 * k4], y.x, acc1);
        acc1 = fmaf(ps[h][4 * k4 + 1], y.y, acc1);
        acc1 = fmaf(ps[h][4 * k4 + 2], y.z, acc1);
        acc1 = fmaf(ps[h][4 * k4 + 3], y.w, acc1);
      }
      o0[h] = o0[h] * al + acc0;
      o1[h] = o1[h] * al + acc1;
    }
    __syncthreads();
  }
  for (int h = 0; h < a.hpg; ++h) {
    const float inv = Lr[h] > 0.0f ? a.v_scale / Lr[h] : 0.0f;  // no visible key: zeros
    store_out(a, row, g * a.hpg + h, lane, o0[h] * inv);
    store_out(a, row, g * a.hpg + h, lane + 64, o1[h] * inv);
    if (a.lse && lane == 0)
      a.lse[(size_t)row * a.H + (size_t)g * a.hpg + h] =
          Lr[h] > 0.0f ? (M[h] + log2f(Lr[h])) * 0.69314718055994531f : -INFINITY;
  }
}

// Launch shape of the MFMA path: waves per workgroup and splits per
// (row, group).  Few units (decode): splits and waves spread a unit's blocks
// over enough workgroups to cover the 256 compute units, each wave still
// taking whole blocks.  Many units (chunked prefill, large batches): one
// wave per unit, so that each CU holds many independent units whose
// memory waits overlap (on the 4,096-row chunk this runs the select +
// attend step 1.4x faster than eight-wave workgroups).
AttendConfig attend_config(const Shape& s) {
  AttendConfig c;
  const int units = s.rows * s.G;
  c.nw = 8;
  c.splits = 1;
  if (s.kv_dtype == kF32) return c;
  if (units >= 512) {
    c.nw = 1;
    return c;
  }
  const int target_wgs = 256;
  int sp = (target_wgs + units - 1) / units;
  sp = max(1, min(sp, (s.K + 3) / 4));
  c.splits = sp;
  const int per_wg = (s.K + sp - 1) / sp;
  c.nw = per_wg >= 8 ? 8 : per_wg >= 4 ? 4 : per_wg >= 2 ? 2 : 1;
  // units * splits <= 510 whenever splits >= 2 (kSplitZoneBytes)
  return c;
}

// [ml: units*S*16*2][o: units*S*16*128] floats; the key-block path's own
// buffers for chunked prefill
size_t attend_workspace_bytes(const Shape& s, const AttendConfig& c) {
  if (k2q_eligible(s)) return k2q_workspace_bytes(s);
  if (c.splits <= 1) return 0;
  const size_t units = (size_t)s.rows * s.G;
  return sizeof(float) * units * c.splits * kHeadsPad * (kDim + 2);
}

// LDS of the fused kernel: the row's keys, its block-table row and a 256-word
// scratch (dynamic), next to the static selection and wave-combine buffers.
static size_t select_dyn_lds(const Shape& s) { return sizeof(uint32_t) * (256 + 2 * (size_t)s.MB); }
static size_t select_static_lds(int nw) {
  const size_t combine = nw > 1 ? (size_t)nw * (8 * 64 * 16 + kHeadsPad * 8) : 0;
  return combine + (size_t)nw * 32 * sizeof(int32_t) + sizeof(GroupSelectLds<8>) + 256;
}

// The fused kernel needs the row's keys in LDS: block tables whose rows fit
// in 64 KB of dynamic LDS, with the whole workgroup inside gfx950's 160 KB.
bool select_fusable(const Shape& s) {
  if (s.kv_dtype == kF32 || k2q_eligible(s)) return false;
  const size_t dyn = select_dyn_lds(s);
  return dyn <= 65536 && dyn + select_static_lds(attend_config(s).nw) <= 160 * 1024;
}

// Workgroups of `kernel` (block threads, lds dynamic bytes) the current
// device holds at once; 0 if the runtime cannot tell.  Cached per kernel.
static long resident_capacity(const void* kernel, int threads, size_t lds) {
  struct Entry {
    const void* k;
    size_t lds;
    int dev;
    long cap;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.k == kernel && e.lds == lds && e.dev == dev) return e.cap;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  cache.push_back(Entry{kernel, lds, dev, (long)per_cu * cus});
  return (long)per_cu * cus;
}

static std::atomic<int> g_spin_limit{kSpinLimit};
void set_merge_spin_limit(int polls) { g_spin_limit.store(polls); }
int merge_spin_limit() { return g_spin_limit.load(); }

// workspace: the split-K partials; status: the workspace's status word.
// zero_partials: the status header and the partials after it are cleared
// first (msa_sparse_attend's layout: header, then partials).
template <int KVT, int NWV, bool SELECT>
static hipError_t launch_kernel(const Shape& s, int splits, const AttendArgs& a, const void* q,
                                const void* kv_data, const void* kv_scales, void* workspace,
                                uint32_t* status, bool zero_partials, hipStream_t st) {
  const int units = s.rows * s.G;
  const void* fn = reinterpret_cast<const void*>(&attend_mfma_kernel<KVT, NWV, SELECT>);
  const size_t lds = SELECT ? select_dyn_lds(s) : 0;
  // the merging workgroup of a split unit waits for the unit's other
  // workgroups: split only when the whole grid can be resident at once
  if (splits > 1 && (long)units * splits > resident_capacity(fn, 64 * NWV, lds)) splits = 1;
  const Partials part =
      make_partials(s, AttendConfig{NWV, splits}, workspace, status, merge_spin_limit());
  if (splits > 1 && zero_partials) {
    const hipError_t e = launch_zero_fill(
        status, kStatusBytes + attend_workspace_bytes(s, AttendConfig{NWV, splits}), st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attend_mfma_kernel<KVT, NWV, SELECT>), dim3(units * splits), dim3(64 * NWV),
                     lds, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint8_t*>(kv_data), static_cast<const uint8_t*>(kv_scales),
                     a, part);
  return hipGetLastError();
}

// zero_partials: clear the split-K partials first (msa_sparse_attend, whose
// workspace carries no zero-fill guarantee); msa_decode's workspace is zero.
template <bool SELECT>
static hipError_t launch_mfma(const Shape& s, const AttendConfig& c, const AttendArgs& a,
                              const void* q, const void* kv_data, const void* kv_scales,
                              void* workspace, uint32_t* status, bool zero_partials,
                              hipStream_t st) {
  if (c.splits < 1 || c.splits > kMaxSplits) return hipErrorInvalidValue;
#define MSA_ATTEND_LAUNCH(KVT, NWV) \
  return launch_kernel<KVT, NWV, SELECT>(s, c.splits, a, q, kv_data, kv_scales, workspace, \
                                         status, zero_partials, st)
  if (s.kv_dtype == kFP8) {
    switch (c.nw) {
      case 1: MSA_ATTEND_LAUNCH(kFP8, 1);
      case 2: MSA_ATTEND_LAUNCH(kFP8, 2);
      case 4: MSA_ATTEND_LAUNCH(kFP8, 4);
      default: MSA_ATTEND_LAUNCH(kFP8, 8);
    }
  } else {
    switch (c.nw) {
      case 1: MSA_ATTEND_LAUNCH(kNVFP4, 1);
      case 2: MSA_ATTEND_LAUNCH(kNVFP4, 2);
      case 4: MSA_ATTEND_LAUNCH(kNVFP4, 4);
      default: MSA_ATTEND_LAUNCH(kNVFP4, 8);
    }
  }
#undef MSA_ATTEND_LAUNCH
}

hipError_t launch_sparse_attend(const Shape& s, const void* q, const void* kv_data,
                                const void* kv_scales, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* q_pos,
                                const int32_t* topk, void* out, float* lse, void* workspace,
                                hipStream_t st) {
  const AttendArgs a = make_attend_args(s, block_table, seq_lens, q_pos, topk, nullptr, nullptr, out, lse);
  if (s.kv_dtype == kF32) {
    hipLaunchKernelGGL(attend_f32_kernel, dim3(s.rows * s.G), dim3(64), 0, st, q,
                       (const float*)kv_data, (int)(s.q_dtype == kBF16), a);
    return hipGetLastError();
  }
  if (k2q_eligible(s))
    return launch_k2q_attend(s, a, q, kv_data, kv_scales, workspace, st);
  uint32_t* status = static_cast<uint32_t*>(workspace);
  return launch_mfma<false>(s, attend_config(s), a, q, kv_data, kv_scales,
                            static_cast<char*>(workspace) + kStatusBytes, status, true, st);
}

hipError_t launch_select_attend(const Shape& s, const void* q, const void* kv_data,
                                const void* kv_scales, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* q_pos,
                                const float* scores, int32_t* topk_out, void* out, float* lse,
                                void* workspace, uint32_t* status, hipStream_t st) {
  AttendArgs a =
      make_attend_args(s, block_table, seq_lens, q_pos, nullptr, scores, topk_out, out, lse);
  return launch_mfma<true>(s, attend_config(s), a, q, kv_data, kv_scales, workspace, status,
                           false, st);
}

}  // namespace msa
