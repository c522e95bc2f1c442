// select_wave.hpp -- block selection by one wavefront, no workgroup barriers.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer"): keep the top-k blocks by pooled index score, the most recent
// block always among them.  The recent block counts inside the k.  The
// indexer's init_blocks / local_blocks settings (vLLM API reference of
// vllm.models.minimax_m3.nvidia.model, the MiniMaxM3SparseAttention
// constructor, which fills them from sparse_init_block / sparse_local_block)
// add more always-kept blocks: read here as
// the first `init` blocks and the last `local` (>= 1, the recent one
// included) blocks of 0..rb, all inside the k.  When rb + 1 > k the free
// candidates are then the contiguous blocks c0 = init .. c1 - 1 with
// c1 = rb + 1 - local, and the k - init - local best of them are kept, ties
// to the lower block index (the host checks init + local <= k, so there are
// more free candidates than places).
//
// Candidates are ordered by the composite key (order-preserving 32-bit key of
// the score, then lower block index), which makes every key distinct.  The
// keys sit in LDS (the caller may have put them there with several waves).
//
// Fast path (need = the number of places left for free candidates): each
// lane, holding candidates l, l+64, ..., takes its best; a 64-lane bitonic
// sort of those gives T0, the need-th best lane maximum.  At least need
// candidates are >= T0, so the need best are all >= T0: only those
// "survivors" can be selected.  They are usually about k; they take slots
// through an LDS counter (order is irrelevant, they are sorted next), a
// second bitonic sort puts the need best in the first lanes and a third
// orders their block ids.  With more than 64 survivors (a strongly
// structured score pattern) a radix select over the bits below the keys'
// common prefix (8-bit digits, LDS histogram, wave scan) finds the need-th
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
// Radix select of the `need` best of keys[0..ncand): writes base + their
// indices to out in ascending order.
__device__ __noinline__ void select_radix(const uint32_t* keys, int ncand, int need,
                                          uint32_t* hist, int32_t* out, int base) {
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
    if (take) out[written + (uint32_t)popc_below(tm, lane)] = base + jj;
    written += (uint32_t)__popcll(tm);
    ties_seen += (uint32_t)__popcll(eqm);
  }
}

// The f-th forced block (f < init + local) of a row whose free candidates
// end at c1: the leading blocks first, then the trailing ones.
__device__ __forceinline__ int forced_block(int f, int init, int c1) {
  return f < init ? f : c1 + (f - init);
}

// Selection from keys already in LDS: keys[0..rb] hold the order keys of
// blocks 0..rb (rb = last visible block, -1 if the row sees no key; the
// forced blocks' keys are not read).  hist: 256 words of LDS scratch.
// Writes K entries to out: ascending block ids, -1 padded.  Must be called
// by all 64 lanes of one wave.
__device__ void wave_select_keys(const uint32_t* keys, int rb, int K, int init, int local,
                                 uint32_t* hist, int32_t* out) {
  const int lane = threadIdx.x & 63;
  if (rb < 0) {  // the row sees no key: nothing to select
    for (int i = lane; i < K; i += 64) out[i] = -1;
    return;
  }
  if (rb + 1 <= K) {
    for (int i = lane; i < K; i += 64) out[i] = i <= rb ? i : -1;
    return;
  }
  const int c0 = init, c1 = rb + 1 - local;
  const int ncand = c1 - c0, need = K - init - local;
  const uint32_t* ck = keys + c0;  // the free candidates
  if (need > 0) {
    // ---- each lane's best, then T0 = the need-th best lane maximum ----
    uint32_t bk = 0u;
    int bi = 0x7FFFFFFF;
    for (int jj = lane; jj < ncand; jj += 64) {
      const uint32_t k = ck[jj];
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
      const uint32_t k = ck[jj];
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
      select_radix(ck, ncand, need, hist, out + init, c0);
    } else {
      uint32_t sk = (uint32_t)lane < total ? hist[lane] : 0u;
      int si = (uint32_t)lane < total ? (int)hist[64 + lane] : 0x7FFFFFFF;
      wave_bitonic<true, 64>(sk, si);  // lanes 0..need-1: the selection (need <= 31)
      if (lane >= need) si = 0x7FFFFFFF;
      wave_bitonic<false, 32>(sk, si);  // ascending block ids in lanes 0..need-1
      if (lane < need) out[init + lane] = c0 + si;
    }
  }
  // forced blocks around the chosen ones keep the row ascending
  if (lane < init) out[lane] = lane;
  if (lane < local) out[init + need + lane] = c1 + lane;
  wave_lds_sync();
}

// Composite candidate: order key in the high word, complemented block index
// in the low word, so that a larger composite is a better candidate (higher
// score, then lower block).  Every candidate's composite is distinct.
__device__ __forceinline__ uint64_t pack_cand(uint32_t key, int idx) {
  return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)idx);
}
__device__ __forceinline__ int cand_index(uint64_t c) { return (int)~(uint32_t)c; }

// Descending bitonic sort over groups of N lanes (N = 32 or 64): lane i of
// a group ends with the group's i-th largest value (for N = 32 the upper
// group of the wave is sorted the other way round and is not used).  Lane
// exchanges are DPP moves and CDNA4 row swaps; the lane-pattern masks are
// compile-time constants, so a stage is an exchange, a max, a min and a
// select.
template <int J>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  return (uint32_t)lane_xor<J>((int)v);
}
template <int J>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v) {
  const uint32_t lo = lane_xor_u32<J>((uint32_t)v);
  const uint32_t hi = lane_xor_u32<J>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// One merge pass of a descending bitonic sort: stages J, J/2, .., 1 of the
// blocks of K lanes.
template <int K, int J, typename T>
__device__ __forceinline__ void sort_desc_merge(T& v) {
  const int lane = threadIdx.x & 63;
  T p;
  if constexpr (sizeof(T) == 8)
    p = lane_xor_u64<J>(v);
  else
    p = lane_xor_u32<J>(v);
  const bool keep_larger = ((lane & J) == 0) == ((lane & K) == 0);
  v = (keep_larger == (p > v)) ? p : v;
  if constexpr (J > 1) sort_desc_merge<K, J / 2>(v);
}

template <int N, int K = 2, typename T>
__device__ __forceinline__ void sort_desc(T& v) {
  sort_desc_merge<K, K / 2>(v);
  if constexpr (K < N) sort_desc<N, K * 2>(v);
}

// Selection by a whole workgroup of NW waves, for a kernel whose threads
// have just loaded the row's keys, thread t the blocks jj with jj % (64 NW)
// == t.  keys[0..rb] in LDS hold the order keys of blocks 0..rb; each
// thread passes the largest key among the free candidates c0 .. c1-1 it
// loaded (0 if none).
//
// The candidates fall into 32 groups: group l holds the blocks loaded by the
// threads at lane positions l and l + 32 of every wave, i.e. the blocks with
// jj % 32 == l.  T0 is the need-th largest group maximum (a 32-lane sort of
// the maxima); the candidates are contiguous and more than need, so at
// least need groups are non-empty and at least need candidates are >= T0:
// the need best all are.  Each wave re-reads its threads' keys and compacts
// its survivors (ballot + mbcnt) into a region of its own.  The survivors,
// usually about k, are gathered into lanes as composites (key, then lower
// block id) and sorted, 32 or 64 lanes wide; the first need lanes hold the
// selection.  All of it runs in registers with lane exchanges; every wave
// computes T0 and the result itself, which saves barriers and broadcasts.
// More than 64 survivors (strongly structured scores) fall back to the
// radix select run by wave 0 over the LDS keys.
//
// On return out_w (this wave's own 32-entry row) holds the K selected block
// ids, -1 padded: the chosen free blocks first, then the forced ones, in an
// order that is the same in every workgroup making this selection (not
// sorted; sort_selection orders a copy).  All LDS writes the threads made
// before the call are visible to the whole workgroup.  Called by every
// thread with workgroup-uniform rb, K <= 32, init and local.
template <int NW>
struct GroupSelectLds {
  uint32_t tmax[64 * NW];    // each thread's largest key
  uint64_t surv[NW][64];     // per wave: the survivors it found
  uint32_t surv_n[NW];
  int32_t radix_out[32];
};

template <int NW>
__device__ __forceinline__ void group_select(const uint32_t* keys, int rb, int K, int init,
                                             int local, uint32_t tmax, GroupSelectLds<NW>& g,
                                             uint32_t* hist, int32_t* out_w) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int c0 = init, c1 = rb + 1 - local;
  const int need = K - init - local;
  if (rb < 0 || rb + 1 <= K || need == 0) {  // nothing to choose
    __syncthreads();
    if (lane < K)
      out_w[lane] = rb < 0 ? -1
                           : (rb + 1 <= K ? (lane <= rb ? lane : -1) : forced_block(lane, init, c1));
    wave_lds_sync();
    return;
  }
  const int ncand = c1 - c0;
  const uint32_t* ck = keys + c0;  // the free candidates
  g.tmax[threadIdx.x] = tmax;
  __syncthreads();
  // ---- T0: the need-th largest of the 32 group maxima; empty groups hold
  // 0, below every real key ----
  uint32_t gm = g.tmax[lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) gm = max(gm, g.tmax[w * 64 + lane]);
  gm = max(gm, (uint32_t)lane_xor<32>((int)gm));
  sort_desc<32>(gm);
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)gm, need - 1);

  // ---- survivors (key >= T0): each wave compacts its own into surv[wave] ----
  constexpr int NT = 64 * NW;
  uint32_t n_w = 0;
  for (int base = 0; base < ncand; base += 8 * NT) {
    uint32_t kk[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) kk[r] = ck[min(base + r * NT + (int)threadIdx.x, ncand - 1)];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int jj = base + r * NT + (int)threadIdx.x;
      const bool s = jj < ncand && kk[r] >= t0;
      const uint64_t m = __ballot(s);
      if (s) {
        const uint32_t slot = n_w + (uint32_t)popc_below(m, lane);
        if (slot < 64) g.surv[wave][slot] = pack_cand(kk[r], jj);
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
    if (wave == 0) select_radix(ck, ncand, need, hist, g.radix_out, c0);
    __syncthreads();
    if (lane < need) out_w[lane] = g.radix_out[lane];
  } else {
    // gather: lane l takes survivor l of the concatenated regions
    uint64_t ci = 0;  // below every real composite
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
    // the need best composites in lanes 0..need-1 (need <= 31)
    if (total <= 32)
      sort_desc<32>(ci);
    else
      sort_desc<64>(ci);
    if (lane < need) out_w[lane] = c0 + cand_index(ci);
  }
  if (lane >= need && lane < K) out_w[lane] = forced_block(lane - need, init, c1);
  wave_lds_sync();
}

// A selection row of K <= 32 entries (block ids and -1 padding, any order)
// in ascending order, padding last: lane l < K returns entry l.  Called by
// all 64 lanes of a wave; `entry` is lane l's entry (lanes >= K: anything).
__device__ __forceinline__ int sort_selection(int entry, int K) {
  const int lane = threadIdx.x & 63;
  uint32_t dummy = 0;
  int v = lane < K && entry >= 0 ? entry : 0x7FFFFFFF;
  wave_bitonic<false, 32>(dummy, v);
  return v == 0x7FFFFFFF ? -1 : v;
}

// Loads the row's scores s[0..n) into LDS as order keys.  All loads of a
// round (PT per thread) are in flight together; the row has MB entries, so
// reading up to n = MB needs no row length.  Called by threads 0..nthreads-1.
template <int PT = 32>
__device__ __forceinline__ void load_keys(const float* __restrict__ s, int n, uint32_t* keys,
                                          int nthreads) {
  const int t = threadIdx.x;
  for (int base = 0; base < n; base += PT * nthreads) {
    float v[PT];
#pragma unroll
    for (int r = 0; r < PT; ++r) v[r] = s[min(base + r * nthreads + t, n - 1)];
#pragma unroll
    for (int r = 0; r < PT; ++r) {
      const int jj = base + r * nthreads + t;
      if (jj < n) keys[jj] = order_key(v[r]);
    }
  }
}

}  // namespace msa
