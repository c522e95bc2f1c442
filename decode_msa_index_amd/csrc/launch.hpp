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
  int q_dtype, iq_dtype, kv_dtype, ik_dtype, out_dtype;
  float sm_scale, index_scale, k_scale, v_scale, ik_scale;
};

// dtype codes (same values as msa_dtype)
constexpr int kF32 = 0, kBF16 = 1, kFP8 = 2, kNVFP4 = 3;

// Split-K partials: per (row, group, split) 16 heads x (m, l) and 16 x 128
// unnormalised outputs, fp32.
constexpr int kHeadsPad = 16;
inline size_t partial_o_floats(const Shape& s) {
  return (size_t)s.rows * s.G * s.K * kHeadsPad * 128;
}
inline size_t partial_ml_floats(const Shape& s) {
  return (size_t)s.rows * s.G * s.K * kHeadsPad * 2;
}

hipError_t launch_index_scores(const Shape& s, const void* index_q, const void* ik_data,
                               const void* ik_scales, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* q_pos,
                               float* scores, hipStream_t st);

hipError_t launch_block_topk(const Shape& s, const float* scores, const int32_t* seq_lens,
                             const int32_t* q_pos, int32_t* topk, hipStream_t st);

hipError_t launch_sparse_attend(const Shape& s, const void* q, const void* kv_data,
                                const void* kv_scales, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* q_pos,
                                const int32_t* topk, void* out, float* lse,
                                int32_t* counters, float* part_o, float* part_ml,
                                hipStream_t st);

}  // namespace msa
