// decode_fused.hip -- the whole decode step (index scan + block max-pool,
// block selection, sparse attention) in one persistent kernel.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer"): the indexer scores every cached block of a query row, the top-k
// blocks (the recent one always among them) are selected per GQA group, and
// attention runs over exactly those blocks.  A row's selection can start as
// soon as that row's blocks are scored, so the kernel overlaps the
// attention of finished rows with the scan of later ones.
//
// Workgroups 0..n_scan-1 scan.  The (row, block) pairs a row can see are
// enumerated row by row (v = 0..V-1) and wave w of the scan takes v = w,
// w + W, w + 2W, ... (W scan waves): every wave gets the same number of
// blocks, and rows complete in order over time.  Each wave prefetches its
// next block while pooling the current one, and writes each block's G
// scores as order keys with device-scope stores (a key is never 0).
//
// Every workgroup (the higher-numbered ones at once, the scanners when they
// are done) then claims attention tasks -- (row, group, split) in row order
// -- from a device-scope ticket counter, and runs attend_task with the
// selection reading the keys: it polls the row's keys until none is 0, which
// needs no completion counter because the data is its own ready flag.  The
// dispatcher starts workgroups in index order, so every scanning workgroup
// is running before any attention workgroup waits on it; the polls are
// bounded all the same.
//
// The workspace must be zero at entry and is zero again at exit: the keys
// are cleared by their last reader, the split-K arrival counters and
// partials by the last arriver, and the ticket by the last failed claim.
#include "attend_task.hpp"
#include "index_block.hpp"
#include "launch.hpp"

namespace msa {

struct FusedArgs {
  IndexArgs x;
  AttendArgs a;
  Partials part;
  const uint16_t* q;
  const uint8_t* kvd;
  const uint8_t* kvs;
  int32_t* ticket;  // claims of attention tasks; zero at entry and at exit
  int rows, n_scan, n_tasks;
};

// Per wave, lane i holds the i-th upcoming block of the wave: its row,
// logical block, last visible key and (clamped) physical block.
struct ScanBatch {
  int row, j, pos, pb;
  bool valid;  // table entry inside the pool
};

// Lanes 0..G-1 publish block b's G scores: as order keys (never 0) with
// device-scope stores, and as floats when the caller takes them.
template <int G>
__device__ __forceinline__ void emit_key(const FusedArgs& f, const ScanBatch& b, float s,
                                         int lane, float* fscores) {
  if (!b.valid) s = -INFINITY;
  if (lane < G) {
    const size_t at = ((size_t)b.row * G + lane) * f.x.MB + b.j;
    __hip_atomic_store(f.a.keys + at, max(order_key(s), 1u), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (fscores) fscores[at] = s;
  }
}

template <int IK, int G>
__device__ __forceinline__ void scan_rows(const FusedArgs& f, const int32_t* pre,
                                          const int32_t* rpos, int V, float* fscores,
                                          uint4* stage) {
  const int lane = threadIdx.x & 63;
  const int W = f.n_scan * 4;
  const int w = blockIdx.x * 4 + wave_id();
  const IndexArgs& x = f.x;
  for (int v0 = w; v0 < V; v0 += 64 * W) {
    // ---- lane i locates block v0 + i*W (binary search of the row prefix) ----
    ScanBatch mine{0, 0, -1, 0, false};
    const int vi = v0 + lane * W;
    const int nb = min(64, (V - v0 + W - 1) / W);  // blocks of this batch
    if (lane < nb) {
      int lo = 0, hi = f.rows;  // pre[lo] <= vi < pre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= vi) lo = mid; else hi = mid;
      }
      mine.row = lo;
      mine.j = vi - pre[lo];
      mine.pos = rpos[lo];
      const int entry = x.bt[(size_t)(lo / x.R) * x.MB + mine.j];
      mine.valid = entry >= 0 && entry < x.P;
      mine.pb = mine.valid ? entry : 0;
    }
    // block i of the batch, read from lane i (wave-uniform values)
    auto at = [&](int i) {
      ScanBatch s;
      s.row = __builtin_amdgcn_readlane(mine.row, i);
      s.j = __builtin_amdgcn_readlane(mine.j, i);
      s.pos = __builtin_amdgcn_readlane(mine.pos, i);
      s.pb = __builtin_amdgcn_readlane(mine.pb, i);
      s.valid = __builtin_amdgcn_readlane((int)mine.valid, i) != 0;
      return s;
    };
    // pipeline unit: a block, as two halves; A and B alternate, so block
    // i+1's loads (and its query) are issued -- and pinned there by a
    // scheduling barrier -- before block i pools: 16 KB in flight per wave.
    // Two blocks per trip keep the buffers in fixed roles; block data is
    // re-read from the batch lanes where needed rather than carried across
    // iterations.
    HalfRaw<IK> a0, a1, b0, b1;
    QueryB qa, qb;
    TileMax tm;
    a0.issue(x, at(0).pb, 0, lane);
    a1.issue(x, at(0).pb, 1, lane);
    load_query_b<G, IK>(x, at(0).row, lane, qa);
    for (int i = 0; i < nb; i += 2) {
      const int i1 = min(i + 1, nb - 1), i2 = min(i + 2, nb - 1);  // past the end: repeats
      b0.issue(x, at(i1).pb, 0, lane);
      b1.issue(x, at(i1).pb, 1, lane);
      load_query_b<G, IK>(x, at(i1).row, lane, qb);
      __builtin_amdgcn_sched_barrier(0);
      tm.init();
      a0.pool(at(i).j, 0, at(i).pos, lane, qa, tm, stage);
      a1.pool(at(i).j, 1, at(i).pos, lane, qa, tm, stage);
      emit_key<G>(f, at(i), finish_block(x, tm), lane, fscores);
      if (i + 1 >= nb) break;
      a0.issue(x, at(i2).pb, 0, lane);
      a1.issue(x, at(i2).pb, 1, lane);
      load_query_b<G, IK>(x, at(i2).row, lane, qa);
      __builtin_amdgcn_sched_barrier(0);
      tm.init();
      b0.pool(at(i1).j, 0, at(i1).pos, lane, qb, tm, stage);
      b1.pool(at(i1).j, 1, at(i1).pos, lane, qb, tm, stage);
      emit_key<G>(f, at(i1), finish_block(x, tm), lane, fscores);
    }
  }
}

// The attention task as a function of its own, so that its register
// allocation does not constrain the scan's.
template <int KV>
__device__ __noinline__ void fused_attend_task(const FusedArgs& f, int t, uint32_t* lds) {
  attend_task<KV, 4, true, true>(f.q, f.kvd, f.kvs, f.a, f.part, t / f.part.S, t % f.part.S, lds);
}

template <int IK, int KV, int G>
__global__ __launch_bounds__(256, 2) void decode_fused_kernel(FusedArgs f, float* fscores) {
  extern __shared__ uint32_t lds[];
  __shared__ int s_ticket;
  const IndexArgs& x = f.x;
  if ((int)blockIdx.x < f.n_scan) {
    // ---- LDS: each wave's staging area, the row prefix of visible blocks and
    // each row's last visible key ----
    uint4* stage = reinterpret_cast<uint4*>(lds) + wave_id() * (kStageBytes / 16);
    int32_t* pre = reinterpret_cast<int32_t*>(lds) + 4 * kStageBytes / 4;  // [rows + 1]
    int32_t* rpos = pre + f.rows + 1;                                      // [rows]
    for (int r = threadIdx.x; r < f.rows; r += blockDim.x) {
      const int pos = row_last_key(x.lens, x.qpos, r, r / x.R, x.MB);
      rpos[r] = pos;
      pre[r + 1] = pos < 0 ? 0 : pos / kBlock + 1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {  // serial prefix: rows are few next to the blocks
      int acc = 0;
      pre[0] = 0;
      for (int r = 1; r <= f.rows; ++r) {
        acc += pre[r];
        pre[r] = acc;
      }
    }
    __syncthreads();
    const int V = pre[f.rows];
    scan_rows<IK, G>(f, pre, rpos, V, fscores, stage);
    if (fscores) {  // the caller's scores past each row's last visible block
      const int W = f.n_scan * 4;
      const int w = blockIdx.x * 4 + wave_id(), lane = threadIdx.x & 63;
      for (int r = w; r < f.rows; r += W) {
        const int first = rpos[r] < 0 ? 0 : rpos[r] / kBlock + 1;
        for (int j = first + lane; j < x.MB; j += 64) {
#pragma unroll
          for (int g = 0; g < G; ++g) fscores[((size_t)r * G + g) * x.MB + j] = -INFINITY;
        }
      }
    }
  }
  // ---- attention tasks, claimed in row order ----
  for (;;) {
    __syncthreads();  // LDS of the previous task (or the scan) is free
    if (threadIdx.x == 0)
      s_ticket = __hip_atomic_fetch_add(f.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = s_ticket;
    if (t >= f.n_tasks) {
      // one failed claim per workgroup: the last one returns the counter to 0
      if (threadIdx.x == 0 && t == f.n_tasks + (int)gridDim.x - 1)
        __hip_atomic_store(f.ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    fused_attend_task<KV>(f, t, lds);
  }
}

// ----------------------------------------------------------------- host ----

template <int IK, int KV, int G>
static hipError_t launch_fused_t(const Shape& s, const FusedArgs& f0, float* fscores,
                                 size_t lds, hipStream_t st) {
  static int g_slots[64];  // resident workgroups per device (occupancy x CUs), 0 = unknown
  auto kern = decode_fused_kernel<IK, KV, G>;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  // occupancy depends on the dynamic LDS; it is computed for the largest
  // size this path admits, so one number serves every call
  if (g_slots[dev] == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, kFusedMaxLds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_slots[dev] = max(1, per_cu) * max(1, cus);
  }
  FusedArgs f = f0;
  const int slots = g_slots[dev];
  // attention workgroups that start at once: enough for a few rows' tasks
  const int n_attn = min(f.n_tasks, max(1, slots / 4));
  f.n_scan = max(1, slots - n_attn);
  hipLaunchKernelGGL(kern, dim3(f.n_scan + n_attn), dim3(256), lds, st, f, fscores);
  return hipGetLastError();
}

bool fused_decode_supported(const Shape& s) {
  if (s.ik_dtype != s.kv_dtype) return false;
  if (s.kv_dtype != kFP8 && s.kv_dtype != kNVFP4) return false;
  if (attend_config(s).nw != 4) return false;
  return fused_lds_bytes(s) <= kFusedMaxLds;
}

size_t fused_lds_bytes(const Shape& s) {
  const size_t attn = sizeof(uint32_t) * (256 + 2 * (size_t)s.MB);
  const size_t scan = 4 * (size_t)kStageBytes + sizeof(int32_t) * (2 * (size_t)s.rows + 1);
  return attn > scan ? attn : scan;
}

hipError_t launch_decode_fused(const Shape& s, const void* index_q, const void* ik_data,
                               const void* ik_scales, const void* q, const void* kv_data,
                               const void* kv_scales, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* q_pos,
                               float* block_scores, uint32_t* keys, int32_t* topk_out,
                               void* out, float* lse, void* attend_ws, int32_t* header,
                               hipStream_t st) {
  FusedArgs f{};
  f.x = IndexArgs{(const uint16_t*)index_q, (const uint8_t*)ik_data, (const uint8_t*)ik_scales,
                  block_table, seq_lens, q_pos, nullptr, s.R, s.MB, s.P,
                  s.index_scale * s.ik_scale};
  const AttendConfig c = attend_config(s);
  f.a = make_attend_args(s, block_table, seq_lens, q_pos, nullptr, nullptr, topk_out, out, lse);
  f.a.keys = keys;
  f.a.clear = keys;
  f.a.spin_limit = kFusedSpinLimit;
  f.a.error = header + 1;
  f.part = make_partials(s, c, attend_ws);
  f.q = (const uint16_t*)q;
  f.kvd = (const uint8_t*)kv_data;
  f.kvs = (const uint8_t*)kv_scales;
  f.ticket = header;
  f.rows = s.rows;
  f.n_tasks = s.rows * s.G * c.splits;
  const size_t lds = fused_lds_bytes(s);
#define MSA_FUSED(IKV, GV) \
  return launch_fused_t<IKV, IKV, GV>(s, f, block_scores, lds, st)
  if (s.kv_dtype == kFP8) {
    switch (s.G) {
      case 1: MSA_FUSED(kFP8, 1);
      case 2: MSA_FUSED(kFP8, 2);
      case 4: MSA_FUSED(kFP8, 4);
      default: MSA_FUSED(kFP8, 8);
    }
  } else {
    switch (s.G) {
      case 1: MSA_FUSED(kNVFP4, 1);
      case 2: MSA_FUSED(kNVFP4, 2);
      case 4: MSA_FUSED(kNVFP4, 4);
      default: MSA_FUSED(kNVFP4, 8);
    }
  }
#undef MSA_FUSED
}

}  // namespace msa
