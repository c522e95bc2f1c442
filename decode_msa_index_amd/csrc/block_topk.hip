// block_topk.hip -- top-k KV-block selection with the most recent block kept.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer"): attention covers the top 16 blocks by pooled index score and
// always keeps the most recent block.  The recent block counts inside the k;
// so do the leading and trailing blocks that the indexer's init_blocks /
// local_blocks settings force (select_wave.hpp states the reading).  The
// rest is the best of the free blocks c0 .. c1-1; ties go to the lower block
// index, which makes the selection unique and deterministic.
//
// Few (row, group) units with long rows (decode batches: a few dozen rows of
// thousands of blocks): one workgroup of four waves per unit runs the
// selection the fused attention kernel runs (group_select), so that the
// chip is not left with one busy wave per unit.  Many units (prefill chunks,
// large batches) or short rows: one wavefront per unit (wave_select_keys).
//
// Rows of more than 16,000 blocks: one 256-thread workgroup per (row,
// group).  The row's scores are read as order-preserving 32-bit keys; the
// best free candidates are found
// as a threshold by radix select on them (4 passes of 8 bits, per-wave LDS
// histograms), then the blocks
// above the threshold and the lowest-indexed ties at the threshold are
// written in ascending order through two block-wide prefix sums.  The work is
// latency-bound (at most a few thousand candidates), not bandwidth-bound.
#include "device.hpp"
#include "launch.hpp"
#include "select_wave.hpp"

namespace msa {

// Exclusive prefix sum over 256 threads; returns the total via *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sm,
                                                         uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t t = sm[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// The row's keys are re-read from global memory in every radix pass (rows
// this long do not fit in LDS).
__global__ __launch_bounds__(256) void block_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ qpos, int32_t* __restrict__ topk, int R, int G, int MB,
    int K, int init, int local) {
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t scan_sm[4];
  __shared__ uint32_t pick[2];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int u = blockIdx.x;
  const int row = u / G, b = row / R;
  const int pos = row_last_key(lens, qpos, row, b, MB);
  int32_t* out = topk + (size_t)u * K;
  const float* s = scores + (size_t)u * MB;
  if (pos < 0) {  // the row sees no key: nothing to select
    for (int i = tid; i < K; i += 256) out[i] = -1;
    return;
  }
  const int rb = pos / kBlock;
  if (rb + 1 <= K) {
    for (int i = tid; i < K; i += 256) out[i] = i <= rb ? i : -1;
    return;
  }
  // forced blocks: 0 .. init-1 lead the row, c1 .. rb end it
  const int c0 = init, c1 = rb + 1 - local, need = K - init - local;
  for (int i = tid; i < init; i += 256) out[i] = i;
  for (int i = tid; i < local; i += 256) out[init + need + i] = c1 + i;
  if (need == 0) return;
  const int ncand = c1 - c0;  // free blocks c0 .. c1-1 compete for `need` places
  const float* sc = s + c0;
  auto key_at = [&](int jj) -> uint32_t { return order_key(sc[jj]); };
  uint32_t prefix = 0, pmask = 0, rem = (uint32_t)need;
  for (int pass = 3; pass >= 0; --pass) {
    const int shift = pass * 8;
    for (int i = tid; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int base = 0; base < ncand; base += 256) {
      const int jj = base + tid;
      const uint32_t key = jj < ncand ? key_at(jj) : 0u;
      const uint32_t dig = (key >> shift) & 255u;
      if (jj < ncand && (key & pmask) == prefix) atomicAdd(&hist[wave][dig], 1u);
    }
    __syncthreads();
    // count of keys whose digit is >= this thread's digit value: scan over
    // digits in descending order (thread t handles digit 255 - t).
    const int dig = 255 - tid;
    const uint32_t cnt = hist[0][dig] + hist[1][dig] + hist[2][dig] + hist[3][dig];
    uint32_t tot;
    const uint32_t above = block_exclusive_scan(cnt, scan_sm, &tot);  // digits > dig
    if (above < rem && above + cnt >= rem) {
      pick[0] = (uint32_t)dig;
      pick[1] = rem - above;
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    pmask |= 0xFFu << shift;
    rem = pick[1];
    __syncthreads();
  }
  // prefix is now the key of the need-th best candidate; `rem` of the
  // candidates equal to it are taken, lowest block index first.
  const int chunk = (ncand + 255) / 256;
  const int j0 = min(tid * chunk, ncand), j1 = min(j0 + chunk, ncand);
  uint32_t n_gt = 0, n_eq = 0;
  for (int jj = j0; jj < j1; ++jj) {
    const uint32_t key = key_at(jj);
    n_gt += key > prefix;
    n_eq += key == prefix;
  }
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan(n_eq, scan_sm, &tot);
  const uint32_t eq_take =
      eq_before >= rem ? 0u : (rem - eq_before < n_eq ? rem - eq_before : n_eq);
  const uint32_t sel_before = block_exclusive_scan(n_gt + eq_take, scan_sm, &tot);
  uint32_t w = sel_before, eq_seen = 0;
  for (int jj = j0; jj < j1; ++jj) {
    const uint32_t key = key_at(jj);
    bool take = key > prefix;
    if (key == prefix) {
      take = eq_seen < eq_take;
      ++eq_seen;
    }
    if (take) out[init + w++] = c0 + jj;
  }
}

constexpr int kWaveSelectMax = 16000;  // keys + histogram stay under 64 KB of LDS

// One unit per workgroup of NW waves: the row's scores as order keys in LDS
// (each thread also keeps the largest key of the free candidates it loaded),
// then the workgroup selection of select_wave.hpp and the ascending store.
template <int NW>
__global__ __launch_bounds__(64 * NW) void block_topk_group_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ qpos, int32_t* __restrict__ topk, int R, int G, int MB,
    int K, int init, int local) {
  extern __shared__ uint32_t lds[];  // [256] scratch, then [MB] keys
  __shared__ GroupSelectLds<NW> gsl;
  __shared__ int32_t sel_w[NW][32];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int u = blockIdx.x, row = u / G, b = row / R;
  const float* s = scores + (size_t)u * MB;
  uint32_t* keys = lds + 256;
  const int pos = row_last_key(lens, qpos, row, b, MB);
  const int rb = pos < 0 ? -1 : pos / kBlock;
  const int c0 = init, c1 = rb + 1 - local;  // the free candidates
  uint32_t tmax = 0u;
  for (int base = 0; base < MB; base += 8 * 64 * NW) {
    float v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = s[min(base + r * 64 * NW + (int)threadIdx.x, MB - 1)];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int jj = base + r * 64 * NW + (int)threadIdx.x;
      if (jj < MB) {
        const uint32_t k = order_key(v[r]);
        keys[jj] = k;
        if (jj >= c0 && jj < c1) tmax = max(tmax, k);
      }
    }
  }
  group_select<NW>(keys, rb, K, init, local, tmax, gsl, lds, sel_w[wave]);
  if (wave == 0) {
    const int v = sort_selection(lane < K ? sel_w[0][lane] : -1, K);
    if (lane < K) topk[(size_t)u * K + lane] = v;
  }
}

// The workgroup form pays where one wave per unit would leave most of the
// chip idle on a long row.
static bool use_group_select(const Shape& s) {
  return s.MB >= 512 && s.MB <= 8064 && (long)s.rows * s.G < 512;
}

__global__ __launch_bounds__(64) void block_topk_wave_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ qpos, int32_t* __restrict__ topk, int R, int G, int MB,
    int K, int init, int local) {
  extern __shared__ uint32_t lds[];  // [256] scratch, then [MB] keys
  const int u = blockIdx.x, row = u / G, b = row / R;
  const float* s = scores + (size_t)u * MB;
  // the first round of score loads does not wait for the row length
  load_keys<16>(s, min(MB, 16 * 64), lds + 256, 64);
  const int pos = row_last_key(lens, qpos, row, b, MB);
  const int rb = pos < 0 ? -1 : pos / kBlock;
  if (rb > 16 * 64) load_keys<16>(s + 16 * 64, rb - 16 * 64, lds + 256 + 16 * 64, 64);
  wave_lds_sync();
  wave_select_keys(lds + 256, rb, K, init, local, lds, topk + (size_t)u * K);
}

hipError_t launch_block_topk(const Shape& s, const float* scores, const int32_t* seq_lens,
                             const int32_t* q_pos, int32_t* topk, hipStream_t st) {
  if (use_group_select(s)) {
    hipLaunchKernelGGL(block_topk_group_kernel<4>, dim3(s.rows * s.G), dim3(256),
                       sizeof(uint32_t) * (256 + s.MB), st, scores, seq_lens, q_pos, topk, s.R,
                       s.G, s.MB, s.K, s.init, s.local);
  } else if (s.MB <= kWaveSelectMax) {
    hipLaunchKernelGGL(block_topk_wave_kernel, dim3(s.rows * s.G), dim3(64),
                       sizeof(uint32_t) * (256 + s.MB), st, scores, seq_lens, q_pos, topk, s.R,
                       s.G, s.MB, s.K, s.init, s.local);
  } else {
    hipLaunchKernelGGL(block_topk_kernel, dim3(s.rows * s.G), dim3(256), 0, st, scores,
                       seq_lens, q_pos, topk, s.R, s.G, s.MB, s.K, s.init, s.local);
  }
  return hipGetLastError();
}

}  // namespace msa
