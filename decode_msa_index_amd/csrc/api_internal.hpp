// api_internal.hpp -- pieces of the C ABI's host side (api.cpp) that other
// translation units of the library call: error reporting, the workspace
// layout and the decode step on a given workspace.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/msa.h"
#include "launch.hpp"

namespace msa_api {

enum Op { kOpIndex = 0, kOpTopk = 1, kOpAttend = 2, kOpDecode = 3, kOpCacheWrite = 4 };

// Records a thread-local message for msa_last_error and returns st.
msa_status fail(msa_status st, const char* fmt, ...);
void clear_error();
// MSA_OK, or MSA_ERR_HIP with the HIP error's text.
msa_status hip_status(hipError_t e, const char* what);

// Workspace regions (byte offsets) of a call: the status header, the split-K
// partials, the pooled scores (msa_decode), and the total.
struct WsLayout {
  size_t status, attend, scores, total;
};
WsLayout ws_layout(const msa_problem* p, int op);

// msa_decode's argument checks (the problem and every pointer but the
// workspace).
msa_status check_decode_args(const msa_problem* p, const void* index_q, const void* ik_data,
                             const void* ik_scales, const void* q, const void* kv_data,
                             const void* kv_scales, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* q_pos,
                             const float* block_scores, const int32_t* topk_idx, const void* out,
                             const float* lse);

// The decode step on workspace ws laid out as w (arguments already checked).
msa_status decode_impl(const msa_problem* p, const void* index_q, const void* ik_data,
                       const void* ik_scales, const void* q, const void* kv_data,
                       const void* kv_scales, const int32_t* block_table,
                       const int32_t* seq_lens, const int32_t* q_pos, float* block_scores,
                       int32_t* topk_idx, void* out, float* lse, char* ws, const WsLayout& w,
                       hipStream_t hs);

// The current device's copy of msa_decode_static's scratch array.
msa_status static_scratch(char** out);

}  // namespace msa_api
