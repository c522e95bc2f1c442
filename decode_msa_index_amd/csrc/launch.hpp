// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernel
// translation units.  Shapes arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

struct Shape {
  int rows;        // B * R query rows
  int R;           // rows per sequence
  int H, G, hpg;   // query heads, groups, heads per group
  int MB, P, K;    // block-table stride, physical blocks, top-k
  int init, local; // forced blocks: the first `init` and the last `local` (>= 1)
  int share;       // sequences per share group of the index scan (1: none)
  int q_dtype, iq_dtype, kv_dtype, ik_dtype, out_dtype;
  float sm_scale, index_scale, k_scale, v_scale, ik_scale;
};

// dtype codes (same values as msa_dtype)
constexpr int kF32 = 0, kBF16 = 1, kFP8 = 2, kNVFP4 = 3;

// Query heads per group are padded to 16 (one MFMA tile).
constexpr int kHeadsPad = 16;
constexpr int kMaxSplits = 8;  // split-K workgroups per (row, group): at most ceil(32 / 4)

hipError_t launch_index_scores(const Shape& s, const void* index_q, const void* ik_data,
                               const void* ik_scales, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* q_pos,
                               float* scores, hipStream_t st);

// Many rows per sequence (chunked prefill): the dense MFMA form of the
// index scan (prefill_index.hip), used by launch_index_scores when supported.
bool prefill_index_supported(const Shape& s);
hipError_t launch_prefill_index_scores(const Shape& s, const void* index_q, const void* ik_data,
                                       const void* ik_scales, const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* q_pos, float* scores, hipStream_t st);

hipError_t launch_block_topk(const Shape& s, const float* scores, const int32_t* seq_lens,
                             const int32_t* q_pos, int32_t* topk, hipStream_t st);

// Attention launch shape: waves per workgroup and workgroups (splits) per
// (row, group).  splits > 1 needs attend_workspace_bytes of scratch.
struct AttendConfig {
  int nw, splits;
};
AttendConfig attend_config(const Shape& s);
size_t attend_workspace_bytes(const Shape& s, const AttendConfig& c);

// Workspace status header: 256 bytes at the front of every workspace that
// holds split-K partials; word 0 becomes non-zero when a merge gives up
// waiting (its partials are then no longer trusted until it is cleared).
constexpr size_t kStatusBytes = 256;
// The split-K partials of every launch shape lie in the first
// kSplitZoneBytes after the status header: attend_config splits a (row,
// group) only below 256 units, into at most ceil(256 / units) workgroups, so
// units * splits <= 510.  This zone (with the header) is the part of a
// workspace that must be zero when a call starts; every call leaves it so.
constexpr size_t kSplitZoneBytes = (size_t)512 * kHeadsPad * (128 + 2) * sizeof(float);  // 128 dims + max + sum

// Polls of one batch of split-K partials before a merger gives up (< 0: the
// merger gives up at once, a test of the failure path).
void set_merge_spin_limit(int polls);
int merge_spin_limit();

// workspace: status header (kStatusBytes) followed by the split-K partials;
// both are cleared before the launch.
hipError_t launch_sparse_attend(const Shape& s, const void* q, const void* kv_data,
                                const void* kv_scales, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* q_pos,
                                const int32_t* topk, void* out, float* lse, void* workspace,
                                hipStream_t st);
// Selection fused into the attention kernel (msa_decode): needs the row's
// block keys in LDS, so only for block tables short enough.  The split-K
// partials in workspace must be zero (they are left zero).
bool select_fusable(const Shape& s);
hipError_t launch_select_attend(const Shape& s, const void* q, const void* kv_data,
                                const void* kv_scales, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* q_pos,
                                const float* scores, int32_t* topk_out, void* out, float* lse,
                                void* workspace, uint32_t* status, hipStream_t st);
// Chunks of many rows per sequence (chunked prefill): the attention grouped
// by key block (k2q_attend.hip).  launch_sparse_attend takes this path when
// k2q_eligible; its workspace is the status header and the split zone, both
// left untouched, then the path's own buffers.
struct AttendArgs;
bool k2q_eligible(const Shape& s);
size_t k2q_workspace_bytes(const Shape& s);
hipError_t launch_k2q_attend(const Shape& s, const AttendArgs& a, const void* q,
                             const void* kv_data, const void* kv_scales, void* workspace,
                             hipStream_t st);
// Quantises new tokens' K, V and index keys into their cache slots
// (cache_write.hip).
hipError_t launch_cache_write(const Shape& s, int num_tokens, const int32_t* token_seq,
                              const int32_t* token_pos, const void* k_new, const void* v_new,
                              const void* ik_new, const int32_t* block_table, void* kv_data,
                              void* kv_scales, void* ik_data, void* ik_scales, hipStream_t st);
// Clears bytes (a multiple of 4) with a fill kernel.
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st);



}  // namespace msa
