// k2q_attend.hip -- sparse attention of a chunk of many query rows, grouped
// by key block.
//
// Method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
// primer": every query head attends exactly its group's selected blocks; the
// vLLM API reference of the MiniMax-M3 model, class MiniMaxM3Model: the
// indexer's top-k buffer is token-major [tokens, index heads, top-k] and is
// inverted by a key-to-query CSR builder, build_k2q_csr, before the sparse
// prefill attention).
//
// A prefill chunk selects the same few hundred blocks of a sequence over and
// over: 4,096 rows over 544 blocks request every (group, block) about 120
// times.  Gathered per (row, group), that is 8.6 GB of K/V for 71 MB of
// distinct blocks, each block dequantised again for every row.  Here the
// selection is inverted instead, and every block is read and dequantised
// once per chunk of up to kChunkRows rows that selected it:
//   1. build:   workgroups over slices of a sequence's rows count the valid
//               entries of topk_idx per (group, block) in LDS histograms,
//               each entry taking its place in its slice's part of the
//               bucket, and store the whole histogram; one workgroup per
//               (sequence, group) adds the slices' counts into bucket starts,
//               each slice's offset in the bucket and a table of work chunks
//               (up to kChunkRows entries of one block each); every entry
//               then lands at bucket start + slice offset + place;
//   2. attend:  one workgroup per chunk stages its block in LDS, K as bf16
//               and V as f16 (both exact); each wave computes one entry at a
//               time -- the entry's (up to 16) heads over that block: S^T =
//               K Q^T and O = P V on MFMA, the block's softmax in fp32 --
//               with the next entry's queries already in flight.  It stores
//               a partial per entry: the output O / l in f16 (O itself for
//               e4m3 V, see kUnnormalised) and (max, sum) in fp32, the sum l
//               being that of the f16 weights the P V product uses (a ninth
//               MFMA tile against ones);
//   3. merge:   one workgroup per (row, group) takes the row's largest
//               partial maximum M, then sums the partials weighted by
//               l 2^(max - M) (2^(max - M) for O) in selection order (fp32),
//               divides by the sum of l 2^(max - M), scales by v_scale
//               and stores the output and lse; each wave a quarter of the
//               dims, with all of its loads in flight at once.
// Which wave takes which entry depends on the order of atomics; the
// arithmetic of an entry and the merge order do not, so the results are
// deterministic.  They differ from a per-row gather by the f16 rounding of
// each block's output (relative 2^-11), which the merge weights by at most 1
// once normalised.
#include "attend_task.hpp"
#include "device.hpp"
#include "launch.hpp"

#include <algorithm>

namespace msa {

constexpr int kChunkRows = 64;  // entries (rows) per work chunk
// Entries a wave attends at once (each operand read from LDS feeds that many
// MFMAs).  Two measured no faster on the 4,096-row chunk: the kernel is bound
// by its HBM traffic, not by LDS.
constexpr int kK2qEntries = 1;
constexpr int kScanThreads = 1024;
constexpr int kCountThreads = 256;
constexpr int kCountPairs = 4;  // entries per thread of a count workgroup
constexpr int kScanBatch = 16;  // slice counts a scan thread loads at once
constexpr size_t kPartialOBytes = (size_t)kHeadsPad * kDim * 2;   // f16 [4][64 lanes][8]
constexpr size_t kPartialMlBytes = (size_t)kHeadsPad * 2 * 4;     // f32 [16 heads][max, sum]
// Rows per sequence from which the grouping pays: measured on a 65,536-token
// context (G = 4, top-16, FP8) against the per-(row, group) kernel, msa_decode
// per step: 182 against 171 us at 512 rows, 230 against 247 us at 768,
// 0.81 against 1.11 ms at 4,096; below the crossover the fixed cost of the
// list build and the merge dominates.
constexpr int kK2qMinRows = 640;
constexpr int kK2qMaxBlocks = 8192;  // the count's LDS histogram of MB words
// The partial output a block leaves: O / l in f16 in general; O itself for
// e4m3 V, where |O| <= (sum of the block's f16 weights, <= 128) * 448 =
// 57,344 fits f16 (65,504) and the same relative rounding is had without a
// multiply per value (the attend kernel's arithmetic adds to its time).
// NVFP4 V reaches 6 * 448 per value, so there O is normalised first.
template <int KV>
constexpr bool kUnnormalised = KV == kFP8;

// Buffers inside the workspace (after its status header and the split zone).  Per (sequence,
// group) bg: entries [bg * R * K, +R * K), chunks [bg * max_chunks, +max_chunks).
struct K2qBufs {
  int32_t* counts;    // [B*G][slices][MB] a slice's entries per block, then its offset
  int32_t* starts;    // [B*G][MB] index of a block's first entry in `entries`
  int32_t* place;     // [pairs] an entry's place in its slice's part of the bucket, -1: not attended
  int32_t* entries;   // [B*G][R*K] entry ids (u * K + slot), grouped by block
  int4* chunks;       // [B*G][max_chunks] (block j, first entry, end, physical block)
  int32_t* nchunks;   // [B*G] chunks in use
  float* ml;          // [pairs][2][16]: the 16 heads' maxima (log2 domain), then sums
  uint4* o;           // [pairs][4][64] of 8 f16
  int max_chunks;     // per (sequence, group)
  int slices;         // count workgroups per (sequence, group)
  int rows_per;       // rows of a slice
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct K2qSizes {
  long long bg, pairs, max_chunks;
};
static K2qSizes k2q_sizes(const Shape& s) {
  K2qSizes z;
  z.bg = (long long)(s.rows / s.R) * s.G;
  z.pairs = (long long)s.rows * s.G * s.K;
  const long long per = (long long)s.R * s.K;  // entries of one (sequence, group)
  z.max_chunks = per / kChunkRows + std::min<long long>(s.MB, per) + 1;
  return z;
}

// Offsets of the buffers from the start of the region; the region's size.
// Rows per count workgroup (a slice) and slices per (sequence, group).
static int k2q_rows_per(const Shape& s) { return std::max(1, kCountThreads * kCountPairs / s.K); }
static int k2q_slices(const Shape& s) { return (s.R + k2q_rows_per(s) - 1) / k2q_rows_per(s); }

static size_t k2q_layout(const Shape& s, size_t off[8]) {
  const K2qSizes z = k2q_sizes(s);
  const size_t sz[8] = {4 * (size_t)(z.bg * k2q_slices(s) * s.MB), 4 * (size_t)(z.bg * s.MB),
                        4 * (size_t)z.pairs,
                        4 * (size_t)z.pairs, 16 * (size_t)(z.bg * z.max_chunks), 4 * (size_t)z.bg,
                        kPartialMlBytes * z.pairs, kPartialOBytes * z.pairs};
  size_t at = 0;
  for (int i = 0; i < 8; ++i) {
    off[i] = at;
    at += align256(sz[i]);
  }
  return at;
}

// Many rows per sequence, an MFMA cache, block tables the build's LDS holds.
bool k2q_eligible(const Shape& s) {
  return (s.kv_dtype == kFP8 || s.kv_dtype == kNVFP4) && s.R >= kK2qMinRows &&
         s.MB <= kK2qMaxBlocks;
}

// After the status header: the split zone, left alone, then the path's own
// buffers.
size_t k2q_workspace_bytes(const Shape& s) {
  size_t off[8];
  return kSplitZoneBytes + k2q_layout(s, off);
}

// The entries the per-row kernels attend: slot sidx below min(K, rb + 1)
// holding a block 0 <= j <= rb whose table entry lies in [0, P).  Returns j,
// or -1.
__device__ __forceinline__ int k2q_entry(const AttendArgs& a, int row, int b, int u, int sidx) {
  const int pos = row_last_key(a.lens, a.qpos, row, b, a.MB);
  const int rb = pos < 0 ? -1 : pos / kBlock;
  if (sidx >= min(a.K, rb + 1)) return -1;
  const int j = a.topk[(size_t)u * a.K + sidx];
  if (j < 0 || j > rb) return -1;
  const int pb = a.bt[(size_t)b * a.MB + j];
  return (pb >= 0 && pb < a.P) ? j : -1;
}

// ---- 1. build ---------------------------------------------------------------------
__device__ __forceinline__ void scan_threads(uint32_t& e, uint32_t& c, uint32_t* sm) {
  // exclusive scans of e and c over the workgroup: wave scans, then the
  // wave totals
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t xe = e, xc = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t ye = __shfl_up(xe, o, 64), yc = __shfl_up(xc, o, 64);
    if (lane >= o) {
      xe += ye;
      xc += yc;
    }
  }
  if (lane == 63) {
    sm[wave] = xe;
    sm[16 + wave] = xc;
  }
  __syncthreads();
  uint32_t be = 0, bc = 0;
  for (int v = 0; v < wave; ++v) {
    be += sm[v];
    bc += sm[16 + v];
  }
  e = be + xe - e;
  c = bc + xc - c;
}

// (sequence, group, slice of rows): LDS histogram per block, each entry's
// place among its slice's entries of that block, the histogram stored whole
// (no atomics outside LDS, nothing to clear first).
__global__ __launch_bounds__(kCountThreads) void k2q_count_kernel(AttendArgs a, K2qBufs w) {
  extern __shared__ int32_t hist[];  // [MB]
  const int tid = threadIdx.x;
  const int bg = blockIdx.x / w.slices, slice = blockIdx.x % w.slices;
  const int b = bg / a.G, g = bg % a.G;
  const int r0 = slice * w.rows_per, r1 = min(a.R, r0 + w.rows_per);
  const int n = max(0, r1 - r0) * a.K;  // <= kCountThreads * kCountPairs
  for (int x = tid; x < a.MB; x += kCountThreads) hist[x] = 0;
  __syncthreads();
  int jj[kCountPairs];
#pragma unroll
  for (int k = 0; k < kCountPairs; ++k) {
    const int i = tid + k * kCountThreads;
    jj[k] = -1;
    if (i < n) {
      const int row = b * a.R + r0 + i / a.K, u = row * a.G + g;
      jj[k] = k2q_entry(a, row, b, u, i % a.K);
    }
  }
#pragma unroll
  for (int k = 0; k < kCountPairs; ++k) {
    const int i = tid + k * kCountThreads;
    const int lp = jj[k] >= 0 ? atomicAdd(&hist[jj[k]], 1) : -1;
    if (i < n) {
      const int row = b * a.R + r0 + i / a.K;
      w.place[((size_t)row * a.G + g) * a.K + i % a.K] = lp;
    }
  }
  __syncthreads();
  int32_t* cnt = w.counts + ((size_t)bg * w.slices + slice) * a.MB;
  for (int x = tid; x < a.MB; x += kCountThreads) cnt[x] = hist[x];
}

// (sequence, group): bucket starts and the table of work chunks.
__global__ __launch_bounds__(kScanThreads) void k2q_scan_kernel(AttendArgs a, K2qBufs w) {
  __shared__ uint32_t sm[32];
  const int tid = threadIdx.x, bg = blockIdx.x;
  int* cnt = w.counts + (size_t)bg * w.slices * a.MB;  // [slices][MB]
  const int per = (a.MB + kScanThreads - 1) / kScanThreads;
  const int x0 = min(a.MB, tid * per), x1 = min(a.MB, x0 + per);
  // each block's total over the slices; each slice's count becomes its
  // offset inside the block's bucket
  uint32_t se = 0, sc = 0;
  for (int x = x0; x < x1; ++x) {
    int n = 0;
    for (int s0 = 0; s0 < w.slices; s0 += kScanBatch) {  // the slices' loads in flight at once
      int c[kScanBatch];
#pragma unroll
      for (int k = 0; k < kScanBatch; ++k)
        c[k] = s0 + k < w.slices ? cnt[(size_t)(s0 + k) * a.MB + x] : 0;
#pragma unroll
      for (int k = 0; k < kScanBatch; ++k) {
        if (s0 + k < w.slices) cnt[(size_t)(s0 + k) * a.MB + x] = n;
        n += c[k];
      }
    }
    w.starts[(size_t)bg * a.MB + x] = n;  // the total, for the pass below
    se += (uint32_t)n;
    sc += ((uint32_t)n + kChunkRows - 1) / kChunkRows;
  }
  scan_threads(se, sc, sm);
  const size_t ebase = (size_t)bg * a.R * a.K;
  const int b = bg / a.G;
  int4* chunks = w.chunks + (size_t)bg * w.max_chunks;
  for (int x = x0; x < x1; ++x) {
    const int n = w.starts[(size_t)bg * a.MB + x];
    const int start = (int)(ebase + se);
    w.starts[(size_t)bg * a.MB + x] = start;
    const int nch = (n + kChunkRows - 1) / kChunkRows;
    // a non-empty bucket's table entry is in [0, P): the count checked it
    const int pb = nch > 0 ? a.bt[(size_t)b * a.MB + x] : 0;
    for (int k = 0; k < nch; ++k)
      chunks[sc + k] = make_int4(x, start + k * kChunkRows, start + min(n, (k + 1) * kChunkRows), pb);
    se += n;
    sc += nch;
  }
  if (tid == kScanThreads - 1) w.nchunks[bg] = (int)sc;  // past every chunk
}

// (32-bit entry indices: the host allows at most 65,535 (row, group) units
// of at most 32 slots.)
__global__ __launch_bounds__(256) void k2q_scatter_kernel(AttendArgs a, K2qBufs w, int pairs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pairs) return;
  const int place = w.place[i];
  if (place < 0) return;
  const int u = i / a.K, row = u / a.G, g = u % a.G, b = row / a.R;
  const int bg = b * a.G + g, slice = (row % a.R) / w.rows_per, j = a.topk[i];
  const int off = w.counts[((size_t)bg * w.slices + slice) * a.MB + j];
  w.entries[w.starts[(size_t)bg * a.MB + j] + off + place] = i;
}

// ---- 2. attend ------------------------------------------------------------------
// LDS: K as bf16 [key][16 chunks of 8 dims], V^T as f16 [dim][16 chunks of 8
// key positions]; chunk c of row r sits at c ^ (r & 15), so that the 16
// lanes of an MFMA operand read (16 rows, one chunk) hit 16 distinct
// 16-byte bank groups.
//
// Operand layout (v_mfma_f32_16x16x32: A lane l holds A[l%16][8(l/16)+e],
// B lane l holds B[8(l/16)+e][l%16], D lane l holds D[4(l/16)+i][l%16]).
// S^T tile t holds keys 16t .. 16t+15 in natural order; in k-step c lane l
// (n = l%16, qd = l/16) holds dims 32qd + 8c .. +7 of both K and Q (the
// contraction order is free as long as the operands agree), and ends with
// keys 16t + 4qd + i of head n.  Its P V operand for key chunk c is the f16
// of tiles 2c and 2c+1: contraction position 32c + 8qd + e stands for key
// 32c + 16(e/4) + 4qd + e%4.  V^T is staged in that position order: within
// each 32-key group, key 16a + 4q + i sits at position 8q + 4a + i.
__device__ __forceinline__ int k_slot(int key, int c) { return key * 16 + (c ^ (key & 15)); }
__device__ __forceinline__ int v_slot(int d, int c) { return d * 16 + (c ^ (d & 15)); }

// Four f16 values of keys t0 .. t0+3 (t0 % 4 == 0) of V^T row d.
__device__ __forceinline__ void v_put4(uint4* v_lds, int d, int t0, uint2 val) {
  const int r = t0 & 31;
  const int c = 4 * (t0 >> 5) + ((r & 15) >> 2);
  reinterpret_cast<uint2*>(v_lds)[2 * v_slot(d, c) + (r >> 4)] = val;
}

__device__ __forceinline__ uint2 f16x4_bits(f16x2 a, f16x2 b) {
  return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// Stages plane (pb, g) of K and of V into LDS: all 64 * NW threads.
template <int KV, int NT>
__device__ __forceinline__ void stage_block(const uint8_t* __restrict__ kvd,
                                            const uint8_t* __restrict__ kvs, size_t kplane,
                                            size_t vplane, uint4* k_lds, uint4* v_lds) {
  const int tid = threadIdx.x;
  if constexpr (KV == kFP8) {
    const uint4* kb = reinterpret_cast<const uint4*>(kvd + kplane * (kBlock * kDim));
    const uint4* vb = reinterpret_cast<const uint4*>(kvd + vplane * (kBlock * kDim));
    constexpr int R = 1024 / NT;  // 16-byte pieces per thread and plane
    uint4 kr[R], vr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kr[r] = kb[tid + r * NT];
      vr[r] = vb[tid + r * NT];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // K piece x: key x/8, dims 16 (x%8) .. +15 -> chunks 2(x%8), 2(x%8)+1
      const int x = tid + r * NT, key = x >> 3, part = x & 7;
      k_lds[k_slot(key, 2 * part)] = __builtin_bit_cast(uint4, fp8x8_bf16(kr[r].x, kr[r].y));
      k_lds[k_slot(key, 2 * part + 1)] = __builtin_bit_cast(uint4, fp8x8_bf16(kr[r].z, kr[r].w));
      // V^T piece x: dim x/8, keys 16 (x%8) .. +15
      const int d = x >> 3, t0 = 16 * (x & 7);
      const uint32_t wv[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v_put4(v_lds, d, t0 + 4 * q,
               f16x4_bits(fp8x2_to_f16x2<false>(wv[q]), fp8x2_to_f16x2<true>(wv[q])));
    }
  } else {
    // NVFP4: data [t][64 B] (K) and [d][64 B] (V^T, keys as nibbles, low
    // nibble first); e4m3 scales K [t][d/16], V [d/16][t]
    const uint4* kb = reinterpret_cast<const uint4*>(kvd + kplane * (kBlock * kDim / 2));
    const uint4* vb = reinterpret_cast<const uint4*>(kvd + vplane * (kBlock * kDim / 2));
    const uint8_t* ks = kvs + kplane * (kBlock * kDim / 16);
    const uint8_t* vs = kvs + vplane * (kBlock * kDim / 16);
    constexpr int R = 512 / NT;
    uint4 kr[R], vr[R], vsc[R][2];
    uint32_t ksc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int x = tid + r * NT;
      kr[r] = kb[x];
      vr[r] = vb[x];
      // K piece x: key x/4, dims 32 (x%4) .. +31: scales 2 (x%4), +1 of the key
      ksc[r] = *reinterpret_cast<const uint16_t*>(ks + (x >> 2) * (kDim / 16) + 2 * (x & 3));
      // V piece x: dim x/4, keys 32 (x%4) .. +31: 32 scale bytes of row d/16
      const uint4* sp = reinterpret_cast<const uint4*>(vs + ((x >> 2) >> 4) * kBlock + 32 * (x & 3));
      vsc[r][0] = sp[0];
      vsc[r][1] = sp[1];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int x = tid + r * NT;
      const int key = x >> 2, part = x & 3;
      const f32x2 sc = fp8x2_to_f32x2<false>(ksc[r]);
      const uint32_t wk[4] = {kr[r].x, kr[r].y, kr[r].z, kr[r].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        k_lds[k_slot(key, 4 * part + c)] = __builtin_bit_cast(uint4, nvfp4x8_bf16(wk[c], sc[c >> 1]));
      const int d = x >> 2, t0 = 32 * part;
      const uint32_t wv[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
      const uint32_t sb[8] = {vsc[r][0].x, vsc[r][0].y, vsc[r][0].z, vsc[r][0].w,
                              vsc[r][1].x, vsc[r][1].y, vsc[r][1].z, vsc[r][1].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // keys t0 + 8m .. +7 with scale bytes 8m .. 8m+7
        const f16x8 h = nvfp4x8_f16(wv[m], sb[2 * m], sb[2 * m + 1]);
        const uint4 hb = __builtin_bit_cast(uint4, h);
        v_put4(v_lds, d, t0 + 8 * m, make_uint2(hb.x, hb.y));
        v_put4(v_lds, d, t0 + 8 * m + 4, make_uint2(hb.z, hb.w));
      }
    }
  }
}

__device__ __forceinline__ f16x8 ones_f16x8() {
  return __builtin_bit_cast(f16x8, make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
}

// The B operand of S^T = K Q^T: head n of the group, dims 32qd + 8c .. +7.
// Lanes past the group's heads load its last head instead (their results
// are never used); the loads are unconditional, so that a wait for them is
// counted exactly.
__device__ __forceinline__ void load_q(const uint16_t* __restrict__ q, const AttendArgs& a,
                                       int row, int g, int n, int qd, bf16x8 (&qo)[4]) {
  const uint4* qp = reinterpret_cast<const uint4*>(
      q + ((size_t)row * a.H + (size_t)g * a.hpg + min(n, a.hpg - 1)) * kDim + qd * 32);
#pragma unroll
  for (int c = 0; c < 4; ++c) qo[c] = __builtin_bit_cast(bf16x8, qp[c]);
}

// Both operands come from LDS for every group of entries: held in registers
// across entries, the block's K operands alone (128 registers) would cut the
// waves per SIMD to one.  A wave takes E entries at a time, so that every
// operand read from LDS feeds E MFMAs.
template <int E>
struct K2qShape {
  static constexpr int waves = E == 1 ? 8 : 4;  // per workgroup; two workgroups per CU (LDS)
  static constexpr int waves_per_simd = E == 1 ? 4 : 2;
};

template <int KV, int E>
__global__ __launch_bounds__(64 * K2qShape<E>::waves)
__attribute__((amdgpu_waves_per_eu(K2qShape<E>::waves_per_simd))) void k2q_attend_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kvd,
    const uint8_t* __restrict__ kvs, AttendArgs a, K2qBufs w) {
  constexpr int NW = K2qShape<E>::waves;
  __shared__ uint4 k_lds[kBlock * 16];
  __shared__ uint4 v_lds[kDim * 16];
  const int bg = blockIdx.x / w.max_chunks, c = blockIdx.x % w.max_chunks;
  // the chunk's descriptor is read together with the count (a slot past the
  // count holds stale bytes and is not used)
  const int nchunks = w.nchunks[bg];
  const int4 ch = w.chunks[(size_t)bg * w.max_chunks + c];
  if (c >= nchunks) return;
  const int j = ch.x, e0 = ch.y, e1 = ch.z, pb = ch.w, g = bg % a.G, b = bg / a.G;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 15, qd = lane >> 4;
  // the wave's entries e0 + wave + NW i, lane i holding entry i's id and
  // last visible key (loaded while the block is staged)
  const int cnt = (e1 - e0 - wave + NW - 1) / NW;
  int my_pair = 0, my_pos = 0;
  if (lane < cnt) {
    my_pair = w.entries[e0 + wave + NW * lane];
    my_pos = row_last_key(a.lens, a.qpos, my_pair / a.K / a.G, b, a.MB);
  }
  // the first group's queries load while the block is staged
  auto q_of = [&](int it0, bf16x8 (&qo)[E][4]) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      load_q(q, a, __shfl(my_pair, min(it0 + e, cnt - 1), 64) / a.K / a.G, g, n, qd, qo[e]);
  };
  bf16x8 qa[E][4], qb[E][4];
  if (cnt > 0) q_of(0, qa);
  stage_block<KV, 64 * NW>(kvd, kvs, ((size_t)pb * 2 + 0) * a.G + g,
                           ((size_t)pb * 2 + 1) * a.G + g, k_lds, v_lds);
  __syncthreads();
  const float cs = a.scale_log2;
  // entries it0 .. it0+E-1 of the wave (past the last: repeats of it, not
  // stored), their queries in qop
  auto attend_group = [&](int it0, const bf16x8 (&qop)[E][4]) {
    // the staged operands are read from LDS again for every group
    asm volatile("" ::: "memory");
    int pair[E], nvalid[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int ii = min(it0 + e, cnt - 1);
      pair[e] = __shfl(my_pair, ii, 64);
      nvalid[e] = min(kBlock, __shfl(my_pos, ii, 64) - j * kBlock + 1);  // >= 1
    }
    // ---- S^T = K Q^T ----
    f32x4 sacc[E][8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int e = 0; e < E; ++e) sacc[e][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8 kk = __builtin_bit_cast(bf16x8, k_lds[k_slot(16 * t + n, 4 * qd + cc)]);
#pragma unroll
        for (int e = 0; e < E; ++e) sacc[e][t] = mfma_bf16(kk, qop[e][cc], sacc[e][t]);
      }
    }
    // ---- each block softmax (head n lives in lanes n, n+16, n+32, n+48):
    // the maximum of the raw dot products, then 2^(s c - m c) with one fma
    // per weight (c > 0 keeps the maximum where it is) ----
    f16x8 pop[E][4];
    float mc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float mraw = -INFINITY;
      if (nvalid[e] == kBlock) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          mraw = fmaxf(mraw, fmaxf(fmaxf(sacc[e][t][0], sacc[e][t][1]),
                                   fmaxf(sacc[e][t][2], sacc[e][t][3])));
      } else {  // the row's own recent block: keys past its position are masked
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = 16 * t + 4 * qd + i < nvalid[e] ? sacc[e][t][i] : -INFINITY;
            sacc[e][t][i] = v;
            mraw = fmaxf(mraw, v);
          }
        }
      }
      mraw = fmaxf(mraw, shfl_xor(mraw, 16));
      mraw = fmaxf(mraw, shfl_xor(mraw, 32));
      mc[e] = mraw * cs;  // the block's maximum, log2 domain
#pragma unroll
      for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pop[e][t >> 1][4 * (t & 1) + i] = (_Float16)exp2_weight(fmaf(sacc[e][t][i], cs, -mc[e]));
      }
    }
    // ---- O = P V, two 16-dim tiles at a time, and the row sums l = P 1
    // (of the same f16 weights) as a ninth tile: they arrive in the output
    // layout, head 4qd+i in every lane of row group qd ----
    f32x4 oacc[E][8], lacc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      lacc[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) lacc[e] = mfma_f16(pop[e][cc], ones_f16x8(), lacc[e]);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if ((dt & 1) == 0) asm volatile("" ::: "memory");
#pragma unroll
      for (int e = 0; e < E; ++e) oacc[e][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const f16x8 vv = __builtin_bit_cast(f16x8, v_lds[v_slot(16 * dt + n, 4 * cc + qd)]);
#pragma unroll
        for (int e = 0; e < E; ++e) oacc[e][dt] = mfma_f16(pop[e][cc], vv, oacc[e][dt]);
      }
    }
    // ---- the partials: O / l of heads 4qd+i, dims 16 dt + n, lane-major;
    // O itself for e4m3 V (see kUnnormalised) ----
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e > 0 && it0 + e >= cnt) break;
      float inv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) inv[i] = kUnnormalised<KV> ? 1.0f : __builtin_amdgcn_rcpf(lacc[e][i]);
      uint4* po = w.o + (size_t)pair[e] * 256;
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2) {
        f16x8 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kUnnormalised<KV>) {
            h[i] = (_Float16)oacc[e][2 * p2][i];
            h[4 + i] = (_Float16)oacc[e][2 * p2 + 1][i];
          } else {
            h[i] = (_Float16)(oacc[e][2 * p2][i] * inv[i]);
            h[4 + i] = (_Float16)(oacc[e][2 * p2 + 1][i] * inv[i]);
          }
        }
        // streaming stores: the partials are read once, by the merge, and
        // should not push the queries out of the caches
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, h),
                                    reinterpret_cast<u32x4_t*>(po + p2 * 64 + lane));
      }
      // (max, sum) record: [16 maxima][16 sums]
      float* pml = w.ml + (size_t)pair[e] * (kHeadsPad * 2);
      if (lane < 16) __builtin_nontemporal_store(mc[e], pml + lane);
      if (n == 0) __builtin_nontemporal_store(lacc[e], reinterpret_cast<f32x4*>(pml + 16) + qd);
    }
  };
  // two query buffers: group it + E's queries load while group it is computed
  for (int it = 0; it < cnt; it += 2 * E) {
    q_of(it + E, qb);
    attend_group(it, qa);
    if (it + E >= cnt) break;
    q_of(it + 2 * E, qa);
    attend_group(it + E, qb);
  }
}

// ---- 3. merge -------------------------------------------------------------------
// One workgroup per (row, group); wave w takes dims 32w .. 32w+31 of all
// 16 heads from every partial (one 16-byte load per lane and partial, all
// issued at once), weighted by l 2^(max - M) and summed in ascending slot
// order, then stores those dims.
template <bool UNNORM>
__global__ __launch_bounds__(256) void k2q_merge_kernel(AttendArgs a, K2qBufs w) {
  __shared__ f32x4 mls[32 * 8];            // the unit's records: [slot][8 x 4 floats]
  __shared__ float ob[4][kHeadsPad][36];   // each wave's 16 heads x 32 dims
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int u = blockIdx.x, row = u / a.G, g = u % a.G;
  const int n = lane & 15, qd = lane >> 4;
  const uint64_t valid =
      __ballot(lane < a.K && w.place[(size_t)u * a.K + min(lane, a.K - 1)] >= 0);
  {  // the K (max, sum) records, 128 bytes each
    const f32x4* src = reinterpret_cast<const f32x4*>(w.ml + (size_t)u * a.K * (kHeadsPad * 2));
    if ((int)threadIdx.x < 8 * a.K) mls[threadIdx.x] = src[threadIdx.x];
  }
  // this wave's 16-byte piece of partials 0 .. 15 (dt = 2 wave, 2 wave + 1),
  // loaded whether or not the slot holds one (the record exists either way;
  // an unused slot's bytes are never read), so that these loads need not
  // wait for the validity bits
  uint4 po[16];
#pragma unroll
  for (int s = 0; s < 16; ++s)
    if (s < a.K) po[s] = load_stream(w.o + ((size_t)u * a.K + s) * 256 + wave * 64 + lane);
  __syncthreads();
  // heads 4qd .. 4qd+3: the largest partial maximum, then the weights
  f32x4 M = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int s = 0; s < a.K; ++s) {
    if ((valid >> s) & 1) {
      const f32x4 m = mls[8 * s + qd];
#pragma unroll
      for (int i = 0; i < 4; ++i) M[i] = fmaxf(M[i], m[i]);
    }
  }
  f32x4 L = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, c0 = L, c1 = L;
  auto add = [&](int s, uint4 piece) {
    const f32x4 m = mls[8 * s + qd], l = mls[8 * s + 4 + qd];
    const f16x8 h = __builtin_bit_cast(f16x8, piece);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the partial's weight: 2^(max - M) on O, l 2^(max - M) on O / l
      const float f = exp2f(m[i] - M[i]), wt = l[i] * f, wo = UNNORM ? f : wt;
      L[i] += wt;
      c0[i] = fmaf((float)h[i], wo, c0[i]);
      c1[i] = fmaf((float)h[4 + i], wo, c1[i]);
    }
  };
#pragma unroll
  for (int s = 0; s < 16; ++s)
    if (s < a.K && ((valid >> s) & 1)) add(s, po[s]);
  for (int s0 = 16; s0 < a.K; s0 += 16) {  // top-k above 16: the next 16 partials
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int s = s0 + k;
      if (s < a.K) po[k] = load_stream(w.o + ((size_t)u * a.K + s) * 256 + wave * 64 + lane);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (s0 + k < a.K && ((valid >> (s0 + k)) & 1)) add(s0 + k, po[k]);
  }
  // heads 4qd+i, dims 32 wave + 16 t + n -> 8 consecutive dims of one head per lane
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float inv = L[i] > 0.0f ? a.v_scale / L[i] : 0.0f;
    ob[wave][4 * qd + i][n] = c0[i] * inv;
    ob[wave][4 * qd + i][16 + n] = c1[i] * inv;
  }
  wave_lds_sync();
  {
    const int h = lane >> 2, d0 = (lane & 3) * 8;
    if (h < a.hpg) {
      const float4 lo = *reinterpret_cast<const float4*>(&ob[wave][h][d0]);
      const float4 hi = *reinterpret_cast<const float4*>(&ob[wave][h][d0 + 4]);
      const float o[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      store_out8(a, row, g * a.hpg + h, 32 * wave + d0, o);
    }
  }
  if (a.lse && wave == 0 && n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * qd + i;
      if (h < a.hpg)
        a.lse[(size_t)row * a.H + (size_t)g * a.hpg + h] =
            L[i] > 0.0f ? (M[i] + log2f(L[i])) * 0.69314718055994531f : -INFINITY;
    }
  }
}

// ---- launch ----------------------------------------------------------------------

// workspace: the status header and the split zone, both left alone (this
// path needs neither and keeps a workspace's merge-failure mark as it is),
// then this path's buffers, which need no clearing.
hipError_t launch_k2q_attend(const Shape& s, const AttendArgs& a, const void* q,
                             const void* kv_data, const void* kv_scales, void* workspace,
                             hipStream_t st) {
  size_t off[8];
  k2q_layout(s, off);
  const K2qSizes z = k2q_sizes(s);
  if (z.pairs == 0) return hipSuccess;
  char* base = static_cast<char*>(workspace) + kStatusBytes + kSplitZoneBytes;
  K2qBufs w;
  w.counts = reinterpret_cast<int32_t*>(base + off[0]);
  w.starts = reinterpret_cast<int32_t*>(base + off[1]);
  w.place = reinterpret_cast<int32_t*>(base + off[2]);
  w.entries = reinterpret_cast<int32_t*>(base + off[3]);
  w.chunks = reinterpret_cast<int4*>(base + off[4]);
  w.nchunks = reinterpret_cast<int32_t*>(base + off[5]);
  w.ml = reinterpret_cast<float*>(base + off[6]);
  w.o = reinterpret_cast<uint4*>(base + off[7]);
  w.max_chunks = (int)z.max_chunks;
  w.rows_per = k2q_rows_per(s);
  w.slices = k2q_slices(s);
  hipLaunchKernelGGL(k2q_count_kernel, dim3((unsigned)(z.bg * w.slices)), dim3(kCountThreads),
                     sizeof(int32_t) * (size_t)s.MB, st, a, w);
  hipLaunchKernelGGL(k2q_scan_kernel, dim3((unsigned)z.bg), dim3(kScanThreads), 0, st, a, w);
  hipLaunchKernelGGL(k2q_scatter_kernel, dim3((unsigned)((z.pairs + 255) / 256)), dim3(256), 0, st,
                     a, w, (int)z.pairs);
  const dim3 agrid((unsigned)(z.bg * z.max_chunks));
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint8_t* kd = static_cast<const uint8_t*>(kv_data);
  const uint8_t* ks = static_cast<const uint8_t*>(kv_scales);
  constexpr int E = kK2qEntries;
  const dim3 ablock(64 * K2qShape<E>::waves);
  if (s.kv_dtype == kFP8)
    hipLaunchKernelGGL((k2q_attend_kernel<kFP8, E>), agrid, ablock, 0, st, qp, kd, ks, a, w);
  else
    hipLaunchKernelGGL((k2q_attend_kernel<kNVFP4, E>), agrid, ablock, 0, st, qp, kd, ks, a, w);
  if (s.kv_dtype == kFP8)
    hipLaunchKernelGGL(k2q_merge_kernel<kUnnormalised<kFP8>>, dim3((unsigned)(s.rows * s.G)),
                       dim3(256), 0, st, a, w);
  else
    hipLaunchKernelGGL(k2q_merge_kernel<kUnnormalised<kNVFP4>>, dim3((unsigned)(s.rows * s.G)),
                       dim3(256), 0, st, a, w);
  return hipGetLastError();
}

}  // namespace msa
