// select_wave.hpp -- block selection by one wavefront, no workgroup barriers.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer"): keep the top-k blocks by pooled index score, the most recent
// block always among them.  The recent block counts inside the k, so the
// rest is the best k-1 of blocks 0..rb-1, ties to the lower block index.
//
// Candidates are ordered by the composite key (order-preserving 32-bit key of
// the score, then lower block index), which makes every key distinct.  The
// keys sit in LDS (the caller may have put them there with several waves).
//
// Fast path: each lane, holding blocks l, l+64, ..., takes its best
// candidate; a 64-lane bitonic sort of those gives T0, the (k-1)-th best lane
// maximum.  At least k-1 candidates are >= T0, so the k-1 best are all >= T0:
// only those "survivors" can be selected.  They are usually about k; they
// take slots through an LDS counter (order is irrelevant, they are sorted
// next), a second bitonic sort puts the k-1 best in the first lanes and a
// third orders their block ids.  With more than 64 survivors (a strongly
// structured score pattern) a radix select over the bits below the keys'
// common prefix (8-bit digits, LDS histogram, wave scan) finds the (k-1)-th
// key and a ballot-based compaction writes the ids.  Lane exchanges use DPP
// and the CDNA4 row-swap instructions, not LDS permutes.
#pragma once

#include "device.hpp"

namespace msa {

// Monotone map float -> uint32 (larger float -> larger key); -0 folds to +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc_below(uint64_t mask, int lane) {
  (void)lane;
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// (key, index) pair order: larger key first, then lower index.
__device__ __forceinline__ bool better(uint32_t ka, int ia, uint32_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ uint32_t wave_reduce_max_u32(uint32_t v) {
  v = max(v, (uint32_t)lane_xor<1>((int)v));
  v = max(v, (uint32_t)lane_xor<2>((int)v));
  v = max(v, (uint32_t)lane_xor<4>((int)v));
  v = max(v, (uint32_t)lane_xor<8>((int)v));
  v = max(v, (uint32_t)lane_xor<16>((int)v));
  return max(v, (uint32_t)lane_xor<32>((int)v));
}
__device__ __forceinline__ uint32_t wave_reduce_min_u32(uint32_t v) {
  v = min(v, (uint32_t)lane_xor<1>((int)v));
  v = min(v, (uint32_t)lane_xor<2>((int)v));
  v = min(v, (uint32_t)lane_xor<4>((int)v));
  v = min(v, (uint32_t)lane_xor<8>((int)v));
  v = min(v, (uint32_t)lane_xor<16>((int)v));
  return min(v, (uint32_t)lane_xor<32>((int)v));
}

// One compare-exchange stage of a bitonic network over the wave: lanes
// paired by lane ^ J; within blocks of K lanes the first lane of a pair gets
// the pair's first element in the order when (lane & K) == 0.
template <bool DESC, int K, int J>
__device__ __forceinline__ void bitonic_stage(uint32_t& key, int& idx) {
  const int lane = threadIdx.x & 63;
  const uint32_t pk = (uint32_t)lane_xor<J>((int)key);
  const int pi = lane_xor<J>(idx);
  const bool want_first = ((lane & J) == 0) == ((lane & K) == 0);
  const bool partner_first = DESC ? better(pk, pi, key, idx) : pi < idx;
  if (partner_first == want_first) {
    key = pk;
    idx = pi;
  }
}

template <bool DESC, int K, int J>
__device__ __forceinline__ void bitonic_merge(uint32_t& key, int& idx) {
  bitonic_stage<DESC, K, J>(key, idx);
  if constexpr (J > 1) bitonic_merge<DESC, K, J / 2>(key, idx);
}

// Bitonic sort of one (key, index) pair per lane over groups of N lanes
// (N = 32 or 64); DESC puts the best pair first, otherwise indices ascend
// (keys ignored).
template <bool DESC, int N, int K = 2>
__device__ __forceinline__ void wave_bitonic(uint32_t& key, int& idx) {
  bitonic_merge<DESC, K, K / 2>(key, idx);
  if constexpr (K < N) wave_bitonic<DESC, N, K * 2>(key, idx);
}

// Radix path.  keys[0..ncand) in LDS; writes out[0..need) ascending.
__device__ __noinline__ void select_radix(const uint32_t* keys, int ncand, int need,
                                          uint32_t* hist, int32_t* out) {
  const int lane = threadIdx.x & 63;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int jj = lane; jj < ncand; jj += 64) {
    kmin = min(kmin, keys[jj]);
    kmax = max(kmax, keys[jj]);
  }
  kmin = wave_reduce_min_u32(kmin);
  kmax = wave_reduce_max_u32(kmax);
  uint32_t prefix, pmask, rem = (uint32_t)need;
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0) {  // every candidate ties: the lowest indices win
    prefix = kmax;
  } else {
    const int hb = 31 - __clz(diff);  // highest bit that differs
    pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    prefix = kmax & pmask;
    for (int top = hb;; top -= 8) {
      const int shift = max(top - 7, 0);
      const uint32_t dmask = (2u << (top - shift)) - 1u;
      for (int i = lane; i < 256; i += 64) hist[i] = 0u;
      wave_lds_sync();
      for (int jj = lane; jj < ncand; jj += 64) {
        const uint32_t key = keys[jj];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
      wave_lds_sync();
      // counts of digits in descending order: lane l holds digits 255-4l .. 252-4l
      uint32_t c[4], local = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[255 - 4 * lane - i];
        local += c[i];
      }
      uint32_t incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
        if (lane >= o) incl += y;
      }
      uint32_t run = incl - local;  // candidates with a larger digit
      int found = -1;
      uint32_t rem_new = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (found < 0 && run < rem && run + c[i] >= rem) {
          found = 255 - 4 * lane - i;
          rem_new = rem - run;
        }
        run += c[i];
      }
      const uint64_t hit = __ballot(found >= 0);
      const int src = hit ? __ffsll((long long)hit) - 1 : 0;  // exactly one lane hits
      const uint32_t digit = (uint32_t)__shfl(found, src, 64);
      rem = (uint32_t)__shfl((int)rem_new, src, 64);
      prefix |= digit << shift;
      pmask |= dmask << shift;
      wave_lds_sync();
      if (shift == 0) break;
    }
  }
  // ascending compaction: keys above T, then the first `rem` ties
  const uint32_t T = prefix;
  uint32_t written = 0, ties_seen = 0;
  for (int c0 = 0; c0 < ncand; c0 += 64) {
    const int jj = c0 + lane;
    const uint32_t key = jj < ncand ? keys[jj] : 0u;
    const bool gt = jj < ncand && key > T;
    const bool eq = jj < ncand && key == T;
    const uint64_t eqm = __ballot(eq);
    const bool take = gt || (eq && ties_seen + (uint32_t)popc_below(eqm, lane) < rem);
    const uint64_t tm = __ballot(take);
    if (take) out[written + (uint32_t)popc_below(tm, lane)] = jj;
    written += (uint32_t)__popcll(tm);
    ties_seen += (uint32_t)__popcll(eqm);
  }
}

// Selection from keys already in LDS: keys[0..rb) hold the order keys of
// blocks 0..rb-1 (rb = last visible block, -1 if the row sees no key).  hist:
// 256 words of LDS scratch.  Writes K entries to out: ascending block ids,
// -1 padded.  Must be called by all 64 lanes of one wave.
__device__ void wave_select_keys(const uint32_t* keys, int rb, int K, uint32_t* hist,
                                 int32_t* out) {
  const int lane = threadIdx.x & 63;
  if (rb < 0) {  // the row sees no key: nothing to select
    for (int i = lane; i < K; i += 64) out[i] = -1;
    return;
  }
  if (rb + 1 <= K) {
    for (int i = lane; i < K; i += 64) out[i] = i <= rb ? i : -1;
    return;
  }
  const int ncand = rb, need = K - 1;
  if (need > 0) {
    // ---- each lane's best, then T0 = the need-th best lane maximum ----
    uint32_t bk = 0u;
    int bi = 0x7FFFFFFF;
    for (int jj = lane; jj < ncand; jj += 64) {
      const uint32_t k = keys[jj];
      if (k > bk) {  // jj ascends: the first maximum has the lowest index
        bk = k;
        bi = jj;
      }
    }
    wave_bitonic<true, 64>(bk, bi);
    const uint32_t tk = (uint32_t)__builtin_amdgcn_readlane((int)bk, need - 1);
    const int ti = __builtin_amdgcn_readlane(bi, need - 1);
    // ---- survivors (not worse than T0) get slots in hist[0..64) / hist[64..128) ----
    uint32_t* cnt = hist + 255;
    if (lane == 0) *cnt = 0u;
    wave_lds_sync();
    for (int jj = lane; jj < ncand; jj += 64) {
      const uint32_t k = keys[jj];
      if (!better(tk, ti, k, jj)) {
        const uint32_t slot = atomicAdd(cnt, 1u);
        if (slot < 64) {
          hist[slot] = k;
          hist[64 + slot] = (uint32_t)jj;
        }
      }
    }
    wave_lds_sync();
    const uint32_t total = *cnt;
    wave_lds_sync();
    if (total > 64) {  // strongly structured scores: take the radix path
      select_radix(keys, ncand, need, hist, out);
    } else {
      uint32_t ck = (uint32_t)lane < total ? hist[lane] : 0u;
      int ci = (uint32_t)lane < total ? (int)hist[64 + lane] : 0x7FFFFFFF;
      wave_bitonic<true, 64>(ck, ci);  // lanes 0..need-1: the selection (need <= 31)
      if (lane >= need) ci = 0x7FFFFFFF;
      wave_bitonic<false, 32>(ck, ci);  // ascending block ids in lanes 0..need-1
      if (lane < need) out[lane] = ci;
    }
  }
  if (lane == 0) out[K - 1] = rb;
  wave_lds_sync();
}

// Composite candidate: order key in the high word, complemented block index
// in the low word, so that a larger composite is a better candidate (higher
// score, then lower block).  Every candidate's composite is distinct.
__device__ __forceinline__ uint64_t pack_cand(uint32_t key, int idx) {
  return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)idx);
}
__device__ __forceinline__ int cand_index(uint64_t c) { return (int)~(uint32_t)c; }
constexpr uint64_t kNoCand = 0x80000000ull;  // pack_cand(0, INT_MAX): below any real candidate

// Number of entries of v[0..n) (LDS, read by all lanes at the same address)
// greater than c.  n is rounded up to a multiple of 8: entries past n must
// hold values that are not greater than any c asked about.
__device__ __forceinline__ int count_greater(const uint64_t* v, int n, uint64_t c) {
  int acc[4] = {0, 0, 0, 0};
  for (int m0 = 0; m0 < n; m0 += 8) {
    uint64_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = v[m0 + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i & 3] += x[i] > c ? 1 : 0;
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Selection by a whole workgroup of NW waves, for a kernel whose threads
// have just loaded the row's keys.  keys[0..rb) in LDS hold the order keys
// of blocks 0..rb-1; each thread passes its best candidate among the blocks
// (< rb) it loaded, as a composite (kNoCand if none).
//
// The candidates fall into 64 groups: group l holds the blocks loaded by the
// threads at lane position l of every wave.  T0 is the (k-1)-th best group
// maximum, found by ranking the 64 maxima by counting.  At least k-1
// candidates are >= T0, so the k-1 best all are: each wave re-reads its
// threads' keys and compacts its survivors (ballot + mbcnt) into a region of
// its own.  The survivors, usually about k, are gathered into lanes, ranked
// by counting (survivor i is chosen when fewer than k-1 survivors beat it)
// and placed by counting smaller block ids, so nothing is sorted.  Every
// wave computes T0 and the result itself, which saves barriers and
// broadcasts.  More than 64 survivors (strongly structured scores) fall back
// to the radix select run by wave 0 over the LDS keys.
//
// On return out_w (this wave's own 32-entry row) holds the K selected block
// ids, ascending, -1 padded, and all LDS writes the threads made before the
// call are visible to the whole workgroup.  Called by every thread with
// workgroup-uniform rb and K <= 32.
template <int NW>
struct GroupSelectLds {
  uint64_t best[64 * NW];    // each thread's best candidate
  uint64_t scratch[NW][64];  // per wave: group maxima, then the gathered survivors
  uint64_t surv[NW][64];     // per wave: the survivors it found
  uint32_t surv_n[NW];
  int32_t radix_out[32];
};

template <int NW>
__device__ void group_select(const uint32_t* keys, int rb, int K, uint64_t mine,
                             GroupSelectLds<NW>& g, uint32_t* hist, int32_t* out_w) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int need = K - 1;
  if (rb < 0 || rb + 1 <= K || need == 0) {  // nothing to choose
    __syncthreads();
    if (lane < K) out_w[lane] = rb < 0 ? -1 : (rb + 1 <= K ? (lane <= rb ? lane : -1) : rb);
    wave_lds_sync();
    return;
  }
  const int ncand = rb;
  g.best[threadIdx.x] = mine;
  __syncthreads();
  // ---- T0: the need-th best of the 64 group maxima ----
  uint64_t gm = g.best[lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) gm = max(gm, g.best[w * 64 + lane]);
  uint64_t* buf = g.scratch[wave];
  buf[lane] = gm;
  wave_lds_sync();
  // groups l < min(64, ncand) hold block l, so ranks 0..need-1 belong to
  // exactly one real group each (empty groups tie at kNoCand below them)
  const uint64_t at = __ballot(count_greater(buf, 64, gm) == need - 1);
  const int src = (int)__builtin_ctzll(at);
  const uint32_t t_lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gm, src);
  const uint32_t t_hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(gm >> 32), src);
  const uint64_t t0 = ((uint64_t)t_hi << 32) | t_lo;

  // ---- survivors (>= T0): each wave compacts its own into surv[wave] ----
  constexpr int NT = 64 * NW;
  uint32_t n_w = 0;
  for (int base = 0; base < ncand; base += 8 * NT) {
    uint32_t kk[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) kk[r] = keys[min(base + r * NT + (int)threadIdx.x, ncand - 1)];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int jj = base + r * NT + (int)threadIdx.x;
      const uint64_t cc = pack_cand(kk[r], jj);
      const bool s = jj < ncand && cc >= t0;
      const uint64_t m = __ballot(s);
      if (s) {
        const uint32_t slot = n_w + (uint32_t)popc_below(m, lane);
        if (slot < 64) g.surv[wave][slot] = cc;
      }
      n_w += (uint32_t)__popcll(m);
    }
  }
  if (lane == 0) g.surv_n[wave] = n_w;
  __syncthreads();
  uint32_t pre[NW], total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    pre[w] = total;
    total += g.surv_n[w];
  }
  if (total > 64) {
    if (wave == 0) select_radix(keys, ncand, need, hist, g.radix_out);
    __syncthreads();
    if (lane < need) out_w[lane] = g.radix_out[lane];
  } else {
    // gather: lane l takes survivor l of the concatenated regions
    uint64_t ci = kNoCand;
    if ((uint32_t)lane < total) {
      int w = 0;
      uint32_t off = (uint32_t)lane;
#pragma unroll
      for (int v = 1; v < NW; ++v) {
        if ((uint32_t)lane >= pre[v]) {
          w = v;
          off = (uint32_t)lane - pre[v];
        }
      }
      ci = g.surv[w][off];
    }
    buf[lane] = ci;
    wave_lds_sync();
    const int rank = count_greater(buf, (int)total, ci);
    const bool chosen = (uint32_t)lane < total && rank < need;
    const uint64_t cm = __ballot(chosen);
    const int j = cand_index(ci);
    // the chosen ids, unordered, then each one's place = smaller chosen ids
    if (chosen) out_w[popc_below(cm, lane)] = j;
    wave_lds_sync();
    int acc[4] = {0, 0, 0, 0};
    for (int m0 = 0; m0 < need; m0 += 8) {
      int x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = out_w[m0 + i];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i & 3] += (m0 + i < need && x[i] < j) ? 1 : 0;
    }
    wave_lds_sync();
    if (chosen) out_w[(acc[0] + acc[1]) + (acc[2] + acc[3])] = j;
  }
  if (lane == 0) out_w[K - 1] = rb;
  wave_lds_sync();
}

// Loads the row's scores s[0..n) into LDS as order keys.  All loads of a
// round (32 per thread) are in flight together; the row has MB entries, so
// reading up to n = MB needs no row length.  Called by threads 0..nthreads-1.
__device__ __forceinline__ void load_keys(const float* __restrict__ s, int n, uint32_t* keys,
                                          int nthreads) {
  const int t = threadIdx.x;
  for (int base = 0; base < n; base += 32 * nthreads) {
    float v[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) v[r] = s[min(base + r * nthreads + t, n - 1)];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int jj = base + r * nthreads + t;
      if (jj < n) keys[jj] = order_key(v[r]);
    }
  }
}

}  // namespace msa
