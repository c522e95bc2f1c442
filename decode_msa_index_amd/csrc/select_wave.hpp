// select_wave.hpp -- block selection by one wavefront, no workgroup barriers.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer"): keep the top-k blocks by pooled index score, the most recent
// block always among them.  The recent block counts inside the k, so the
// rest is the best k-1 of blocks 0..rb-1, ties to the lower block index.
//
// Candidates are ordered by the composite key (order-preserving 32-bit key of
// the score, then lower block index), which makes every key distinct.
//
// Fast path (wave_select): the candidates stay in registers, lane l holding
// blocks l, l+64, ...  Each lane takes its best candidate; a 64-lane bitonic
// sort of those gives T0, the (k-1)-th best lane maximum.  At least k-1
// candidates are >= T0, so the k-1 best are all >= T0: only those
// "survivors" can be selected.  They are usually about k, at most 64 are
// compacted through LDS and sorted by a second bitonic sort, whose first k-1
// lanes are the answer; a third sort orders their block ids.  No atomics and
// no workgroup barriers.  With more than 64 survivors (a strongly structured
// score pattern) it falls back to wave_select_radix: a radix select over the
// bits below the keys' common prefix (8-bit digits, LDS histogram, wave scan)
// and a ballot-based compaction.
#pragma once

#include "device.hpp"

namespace msa {

// Monotone map float -> uint32 (larger float -> larger key); -0 folds to +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Keeps the compiler from moving LDS accesses across this point; the
// hardware already executes a wave's LDS operations in order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ int popc_below(uint64_t mask, int lane) {
  return __popcll(mask & ((1ull << lane) - 1ull));
}

// Radix-select version (any candidate distribution).  s: the row's pooled
// scores (rb+1 valid entries), rb: last visible block (-1: the row sees no
// key), keys: LDS scratch of at least max(rb, 0) words, hist: LDS scratch of
// 256 words.  Writes K entries to out (global or LDS): ascending block ids,
// -1 padded.  Must be called by all 64 lanes of one wave.
template <typename OutT>
__device__ void wave_select_radix(const float* __restrict__ s, int rb, int K, uint32_t* keys,
                                  uint32_t* hist, OutT* out) {
  const int lane = threadIdx.x & 63;
  if (rb < 0) {  // the row sees no key: nothing to select
    for (int i = lane; i < K; i += 64) out[i] = -1;
    return;
  }
  if (rb + 1 <= K) {
    for (int i = lane; i < K; i += 64) out[i] = i <= rb ? i : -1;
    return;
  }
  if (K == 1) {
    if (lane == 0) out[0] = rb;
    return;
  }
  const int ncand = rb;  // blocks 0..rb-1 compete for k-1 places
  const uint32_t need = (uint32_t)(K - 1);

  // ---- keys into LDS, 16 loads in flight per lane per round ----
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int base = 0; base < ncand; base += 16 * 64) {
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jj = base + r * 64 + lane;
      v[r] = jj < ncand ? s[jj] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jj = base + r * 64 + lane;
      if (jj < ncand) {
        const uint32_t k = order_key(v[r]);
        keys[jj] = k;
        kmin = min(kmin, k);
        kmax = max(kmax, k);
      }
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  wave_lds_sync();

  // ---- radix select below the common prefix ----
  uint32_t prefix, pmask, rem = need;
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0) {  // every candidate ties: the lowest indices win
    prefix = kmax;
    pmask = 0xFFFFFFFFu;
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

  // ---- ascending compaction: keys above T, then the first `rem` ties ----
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
  if (lane == 0) out[K - 1] = rb;
}

// (key, index) pair order: larger key first, then lower index.
__device__ __forceinline__ bool better(uint32_t ka, int ia, uint32_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Value of lane (lane ^ J).  J = 1, 2, 8 are single DPP moves (quad
// permutes, rotate a 16-lane row by 8); J = 4 takes the lane 4 up or down
// with two DPP row shifts; 16 and 32 cross rows through ds_bpermute.
template <int J>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);  // row_shl:4
    const int dn = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else {
    return __shfl_xor(v, J, 64);
  }
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

// Selects for one (row, group); see the header comment.  Same contract as
// wave_select_radix; rows of more than 64*RMAX candidates go to it directly.
template <int RMAX, typename OutT>
__device__ void wave_select(const float* __restrict__ s, int rb, int K, uint32_t* keys,
                            uint32_t* hist, OutT* out) {
  const int lane = threadIdx.x & 63;
  const int ncand = rb;  // blocks 0..rb-1 compete for k-1 places
  if (rb < 0 || rb + 1 <= K || K == 1 || ncand > 64 * RMAX) {
    wave_select_radix(s, rb, K, keys, hist, out);
    return;
  }
  const int need = K - 1;
  // ---- candidates into registers: unconditional (clamped) loads, so that
  // all of them are in flight together ----
  float v[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) v[r] = s[min(r * 64 + lane, ncand - 1)];
  uint32_t kr[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) kr[r] = r * 64 + lane < ncand ? order_key(v[r]) : 0u;
  // ---- each lane's best, then T0 = the need-th best lane maximum ----
  uint32_t bk = 0u;
  int bi = 0x7FFFFFFF;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int jj = r * 64 + lane;
    if (jj < ncand && kr[r] > bk) {  // r ascends: first maximum = lowest index
      bk = kr[r];
      bi = jj;
    }
  }
  wave_bitonic<true, 64>(bk, bi);
  const uint32_t tk = (uint32_t)__shfl((int)bk, need - 1, 64);
  const int ti = __shfl(bi, need - 1, 64);
  // ---- survivors: candidates not worse than T0 ----
  int mine = 0;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int jj = r * 64 + lane;
    mine += (jj < ncand && !better(tk, ti, kr[r], jj)) ? 1 : 0;
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int total = __shfl(incl, 63, 64);
  if (total > 64) {
    wave_select_radix(s, rb, K, keys, hist, out);
    return;
  }
  // compact survivors (key, index) into LDS: keys[0..total), hist[0..total)
  int w = incl - mine;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    const int jj = r * 64 + lane;
    if (jj < ncand && !better(tk, ti, kr[r], jj)) {
      keys[w] = kr[r];
      hist[w] = (uint32_t)jj;
      ++w;
    }
  }
  wave_lds_sync();
  uint32_t ck = lane < total ? keys[lane] : 0u;
  int ci = lane < total ? (int)hist[lane] : 0x7FFFFFFF;
  wave_bitonic<true, 64>(ck, ci);  // lanes 0..need-1: the selection (need <= 31)
  if (lane >= need) ci = 0x7FFFFFFF;
  wave_bitonic<false, 32>(ck, ci);  // ascending block ids in lanes 0..need-1
  if (lane < need) out[lane] = ci;
  if (lane == 0) out[K - 1] = rb;
  wave_lds_sync();
}

}  // namespace msa
