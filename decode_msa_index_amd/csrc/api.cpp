// api.cpp -- the C ABI declared in include/msa.h: host-side validation, then
// launches on the caller's stream.  No allocation, no state across calls
// (apart from the merge spin limit, a test hook).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "api_internal.hpp"

namespace msa_api {

thread_local char g_err[512] = "";

void clear_error() { g_err[0] = '\0'; }

msa_status fail(msa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;

msa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSA_OK;
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

msa::Shape shape_of(const msa_problem* p) {
  msa::Shape s;
  s.rows = p->num_seqs * p->rows_per_seq;
  s.R = p->rows_per_seq;
  s.H = p->num_q_heads;
  s.G = p->num_kv_groups;
  s.hpg = p->num_q_heads / p->num_kv_groups;
  s.MB = p->max_blocks_per_seq;
  s.P = p->num_phys_blocks;
  s.K = p->top_k;
  s.init = p->init_blocks;
  s.local = p->local_blocks > 1 ? p->local_blocks : 1;
  s.share = p->share_seqs > 1 ? p->share_seqs : 1;
  s.q_dtype = p->q_dtype;
  s.iq_dtype = p->index_q_dtype;
  s.kv_dtype = p->kv_dtype;
  s.ik_dtype = p->index_k_dtype;
  s.out_dtype = p->out_dtype;
  s.sm_scale = p->sm_scale;
  s.index_scale = p->index_scale;
  s.k_scale = p->k_scale;
  s.v_scale = p->v_scale;
  s.ik_scale = p->index_k_scale;
  return s;
}

// Device scratch.  msa_sparse_attend needs room for the split-K partial
// states when it splits a (row, group) over several workgroups, behind a
// status header; msa_decode needs the header and the partials, then the
// pooled scores.
WsLayout ws_layout(const msa_problem* p, int op) {
  WsLayout w{};
  if (op != kOpAttend && op != kOpDecode) return w;
  const msa::Shape s = shape_of(p);
  const size_t attend = round_up(msa::attend_workspace_bytes(s, msa::attend_config(s)));
  if (op == kOpAttend && attend == 0) return w;
  w.status = 0;
  w.attend = msa::kStatusBytes;
  w.scores = w.attend + attend;
  w.total = w.scores;
  if (op == kOpDecode) {
    // the pooled scores lie past the split zone, which every call leaves
    // zero: they need no clearing after use
    w.scores = std::max(w.scores, msa::kStatusBytes + msa::kSplitZoneBytes);
    w.total = w.scores + round_up(sizeof(float) * (size_t)s.rows * s.G * s.MB);
  }
  return w;
}

bool pos_finite(float x) { return std::isfinite(x) && x > 0.0f; }

}  // namespace msa_api

using namespace msa_api;

extern "C" {

msa_status msa_check_problem(const msa_problem* p, int32_t op) {
  clear_error();
  if (!p) return fail(MSA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (op < kOpIndex || op > kOpCacheWrite) return fail(MSA_ERR_INVALID_ARGUMENT, "unknown op %d", op);
  if (p->num_seqs < 0) return fail(MSA_ERR_INVALID_ARGUMENT, "num_seqs < 0");
  if (p->rows_per_seq < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "rows_per_seq < 1");
  if (p->num_kv_groups < 1 || p->num_q_heads < 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "num_kv_groups and num_q_heads must be >= 1");
  if (p->num_q_heads % p->num_kv_groups)
    return fail(MSA_ERR_INVALID_ARGUMENT, "num_q_heads %% num_kv_groups != 0");
  if (p->max_blocks_per_seq < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq < 1");
  if (p->num_phys_blocks < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "num_phys_blocks < 1");
  if (p->top_k < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "top_k < 1");
  const long long rows = (long long)p->num_seqs * p->rows_per_seq;
  if (rows * p->num_kv_groups > 65535)
    return fail(MSA_ERR_UNSUPPORTED, "num_seqs * rows_per_seq * num_kv_groups > 65535");
  if ((long long)p->max_blocks_per_seq * 128 > (1LL << 30))
    return fail(MSA_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size > 2^30 tokens");
  if (p->head_dim != 128 || p->index_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "head_dim and index_dim must be 128");
  if (p->block_size != 128) return fail(MSA_ERR_UNSUPPORTED, "block_size must be 128");
  if (p->top_k > 32) return fail(MSA_ERR_UNSUPPORTED, "top_k must be <= 32");
  if (p->init_blocks < 0 || p->local_blocks < 0)
    return fail(MSA_ERR_INVALID_ARGUMENT, "init_blocks and local_blocks must be >= 0");
  if ((long long)p->init_blocks + (p->local_blocks > 1 ? p->local_blocks : 1) > p->top_k)
    return fail(MSA_ERR_INVALID_ARGUMENT,
                "init_blocks + max(local_blocks, 1) > top_k: the forced blocks do not fit");
  if (p->share_seqs < 0 || p->share_seqs > 64)
    return fail(MSA_ERR_INVALID_ARGUMENT, "share_seqs must be in [0, 64]");
  if (p->share_seqs > 1 && p->rows_per_seq != 1)
    return fail(MSA_ERR_UNSUPPORTED, "share_seqs > 1 needs rows_per_seq == 1");
  const int G = p->num_kv_groups, hpg = p->num_q_heads / p->num_kv_groups;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(MSA_ERR_UNSUPPORTED, "num_kv_groups must be 1, 2, 4 or 8");
  if (hpg > 16) return fail(MSA_ERR_UNSUPPORTED, "more than 16 query heads per group");
  const bool need_index = op == kOpIndex || op == kOpDecode || op == kOpCacheWrite;
  const bool need_attend = op == kOpAttend || op == kOpDecode || op == kOpCacheWrite;
  if (need_index) {
    const int ik = p->index_k_dtype, iq = p->index_q_dtype;
    if (ik == MSA_DTYPE_FP8_E4M3 || ik == MSA_DTYPE_NVFP4) {
      if (iq != MSA_DTYPE_BF16)
        return fail(MSA_ERR_UNSUPPORTED, "fp8/nvfp4 index keys need bf16 index queries");
    } else if (ik == MSA_DTYPE_F32) {
      if (iq != MSA_DTYPE_F32)
        return fail(MSA_ERR_UNSUPPORTED, "f32 index keys need f32 index queries");
    } else {
      return fail(MSA_ERR_UNSUPPORTED, "index_k_dtype %d not supported", ik);
    }
    if (!pos_finite(p->index_scale) || !pos_finite(p->index_k_scale))
      return fail(MSA_ERR_INVALID_ARGUMENT, "index_scale and index_k_scale must be finite and > 0");
  }
  if (need_attend) {
    const int kv = p->kv_dtype, q = p->q_dtype;
    if (kv == MSA_DTYPE_FP8_E4M3 || kv == MSA_DTYPE_NVFP4) {
      if (q != MSA_DTYPE_BF16) return fail(MSA_ERR_UNSUPPORTED, "fp8/nvfp4 K/V need bf16 queries");
    } else if (kv == MSA_DTYPE_F32) {
      if (q != MSA_DTYPE_F32 && q != MSA_DTYPE_BF16)
        return fail(MSA_ERR_UNSUPPORTED, "q_dtype %d not supported", q);
    } else {
      return fail(MSA_ERR_UNSUPPORTED, "kv_dtype %d not supported", kv);
    }
    if (p->out_dtype != MSA_DTYPE_BF16 && p->out_dtype != MSA_DTYPE_F32)
      return fail(MSA_ERR_UNSUPPORTED, "out_dtype must be bf16 or f32");
    if (!pos_finite(p->sm_scale) || !pos_finite(p->k_scale) || !std::isfinite(p->v_scale))
      return fail(MSA_ERR_INVALID_ARGUMENT, "sm_scale, k_scale must be finite and > 0; v_scale finite");
  }
  return MSA_OK;
}

msa_status msa_workspace_bytes(const msa_problem* p, int32_t op, size_t* bytes) {
  if (!bytes) return fail(MSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  msa_status st = msa_check_problem(p, op);
  if (st != MSA_OK) return st;
  *bytes = ws_layout(p, op).total;
  return MSA_OK;
}

#define REQUIRE(ptr, align)                                                          \
  do {                                                                               \
    if (!(ptr)) return fail(MSA_ERR_INVALID_ARGUMENT, "%s is NULL", #ptr);           \
    if (!aligned((ptr), (align)))                                                    \
      return fail(MSA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", #ptr, (int)(align)); \
  } while (0)

#define OPTIONAL(ptr, align)                                                         \
  do {                                                                               \
    if ((ptr) && !aligned((ptr), (align)))                                           \
      return fail(MSA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", #ptr, (int)(align)); \
  } while (0)

static msa_status check_index_args(const msa_problem* p, const void* index_q,
                                   const void* ik_data, const void* ik_scales,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* q_pos) {
  REQUIRE(index_q, 16);
  REQUIRE(ik_data, 16);
  if (p->index_k_dtype == MSA_DTYPE_NVFP4) REQUIRE(ik_scales, 16);
  REQUIRE(block_table, 4);
  REQUIRE(seq_lens, 4);
  OPTIONAL(q_pos, 4);
  if (!q_pos && p->rows_per_seq != 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "q_pos is required when rows_per_seq > 1");
  return MSA_OK;
}

static msa_status check_attend_args(const msa_problem* p, const void* q, const void* kv_data,
                                    const void* kv_scales, const int32_t* block_table,
                                    const int32_t* seq_lens, const int32_t* q_pos,
                                    const void* out, const float* lse) {
  REQUIRE(q, 16);
  REQUIRE(kv_data, 16);
  if (p->kv_dtype == MSA_DTYPE_NVFP4) REQUIRE(kv_scales, 16);
  REQUIRE(block_table, 4);
  REQUIRE(seq_lens, 4);
  OPTIONAL(q_pos, 4);
  REQUIRE(out, 16);
  OPTIONAL(lse, 4);
  if (!q_pos && p->rows_per_seq != 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "q_pos is required when rows_per_seq > 1");
  return MSA_OK;
}


msa_status msa_index_scores(const msa_problem* p, const void* index_q, const void* ik_data,
                            const void* ik_scales, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* q_pos,
                            float* block_scores, void* stream) {
  msa_status st = msa_check_problem(p, kOpIndex);
  if (st != MSA_OK) return st;
  st = check_index_args(p, index_q, ik_data, ik_scales, block_table, seq_lens, q_pos);
  if (st != MSA_OK) return st;
  REQUIRE(block_scores, 4);
  if (p->num_seqs == 0) return MSA_OK;
  const msa::Shape s = shape_of(p);
  return hip_status(msa::launch_index_scores(s, index_q, ik_data, ik_scales, block_table,
                                             seq_lens, q_pos, block_scores,
                                             (hipStream_t)stream),
                    "index scores launch");
}

msa_status msa_block_topk(const msa_problem* p, const float* block_scores,
                          const int32_t* seq_lens, const int32_t* q_pos, int32_t* topk_idx,
                          void* stream) {
  msa_status st = msa_check_problem(p, kOpTopk);
  if (st != MSA_OK) return st;
  REQUIRE(block_scores, 4);
  REQUIRE(seq_lens, 4);
  OPTIONAL(q_pos, 4);
  REQUIRE(topk_idx, 4);
  if (!q_pos && p->rows_per_seq != 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "q_pos is required when rows_per_seq > 1");
  if (p->num_seqs == 0) return MSA_OK;
  const msa::Shape s = shape_of(p);
  return hip_status(msa::launch_block_topk(s, block_scores, seq_lens, q_pos, topk_idx,
                                           (hipStream_t)stream),
                    "block top-k launch");
}

msa_status msa_sparse_attend(const msa_problem* p, const void* q, const void* kv_data,
                             const void* kv_scales, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* q_pos,
                             const int32_t* topk_idx, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  msa_status st = msa_check_problem(p, kOpAttend);
  if (st != MSA_OK) return st;
  st = check_attend_args(p, q, kv_data, kv_scales, block_table, seq_lens, q_pos, out, lse);
  if (st != MSA_OK) return st;
  REQUIRE(topk_idx, 4);
  const WsLayout w = ws_layout(p, kOpAttend);
  if (w.total) {
    REQUIRE(workspace, kAlign);
    if (workspace_bytes < w.total)
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                  workspace_bytes, w.total);
  } else {
    OPTIONAL(workspace, kAlign);
  }
  if (p->num_seqs == 0) return MSA_OK;
  const msa::Shape s = shape_of(p);
  return hip_status(msa::launch_sparse_attend(s, q, kv_data, kv_scales, block_table,
                                              seq_lens, q_pos, topk_idx, out, lse,
                                              static_cast<char*>(workspace) + w.status,
                                              (hipStream_t)stream),
                    "sparse attend launch");
}

}  // extern "C"

namespace msa_api {

// The decode step on a workspace the caller (or the library's static scratch)
// provides; arguments already validated.
msa_status decode_impl(const msa_problem* p, const void* index_q, const void* ik_data,
                              const void* ik_scales, const void* q, const void* kv_data,
                              const void* kv_scales, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* q_pos, float* block_scores,
                              int32_t* topk_idx, void* out, float* lse, char* ws,
                              const WsLayout& w, hipStream_t hs) {
  const msa::Shape s = shape_of(p);
  void* aws = ws + w.attend;
  uint32_t* status = reinterpret_cast<uint32_t*>(ws + w.status);
  float* scores = block_scores ? block_scores : reinterpret_cast<float*>(ws + w.scores);
  msa_status st;
  if (msa::select_fusable(s)) {
    // two launches: the index scan, then selection + attention in one kernel
    st = hip_status(msa::launch_index_scores(s, index_q, ik_data, ik_scales, block_table,
                                             seq_lens, q_pos, scores, hs),
                    "index scores launch");
    if (st != MSA_OK) return st;
    return hip_status(msa::launch_select_attend(s, q, kv_data, kv_scales, block_table, seq_lens,
                                                q_pos, scores, topk_idx, out, lse, aws, status,
                                                hs),
                      "select + attend launch");
  }
  // three kernels
  st = hip_status(msa::launch_index_scores(s, index_q, ik_data, ik_scales, block_table,
                                           seq_lens, q_pos, scores, hs),
                  "index scores launch");
  if (st != MSA_OK) return st;
  st = hip_status(msa::launch_block_topk(s, scores, seq_lens, q_pos, topk_idx, hs),
                  "block top-k launch");
  if (st != MSA_OK) return st;
  return hip_status(msa::launch_sparse_attend(s, q, kv_data, kv_scales, block_table, seq_lens,
                                              q_pos, topk_idx, out, lse, ws + w.status, hs),
                    "sparse attend launch");
}

msa_status check_decode_args(const msa_problem* p, const void* index_q,
                                    const void* ik_data, const void* ik_scales, const void* q,
                                    const void* kv_data, const void* kv_scales,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* q_pos, const float* block_scores,
                                    const int32_t* topk_idx, const void* out, const float* lse) {
  msa_status st = msa_check_problem(p, kOpDecode);
  if (st != MSA_OK) return st;
  st = check_index_args(p, index_q, ik_data, ik_scales, block_table, seq_lens, q_pos);
  if (st != MSA_OK) return st;
  st = check_attend_args(p, q, kv_data, kv_scales, block_table, seq_lens, q_pos, out, lse);
  if (st != MSA_OK) return st;
  OPTIONAL(block_scores, 4);
  REQUIRE(topk_idx, 4);
  return MSA_OK;
}

}  // namespace msa_api

extern "C" {

msa_status msa_decode(const msa_problem* p, const void* index_q, const void* ik_data,
                      const void* ik_scales, const void* q, const void* kv_data,
                      const void* kv_scales, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* q_pos, float* block_scores,
                      int32_t* topk_idx, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  msa_status st = check_decode_args(p, index_q, ik_data, ik_scales, q, kv_data, kv_scales,
                                    block_table, seq_lens, q_pos, block_scores, topk_idx, out,
                                    lse);
  if (st != MSA_OK) return st;
  const WsLayout w = ws_layout(p, kOpDecode);
  REQUIRE(workspace, kAlign);
  if (workspace_bytes < w.total)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                workspace_bytes, w.total);
  if (p->num_seqs == 0) return MSA_OK;
  return decode_impl(p, index_q, ik_data, ik_scales, q, kv_data, kv_scales, block_table,
                     seq_lens, q_pos, block_scores, topk_idx, out, lse,
                     static_cast<char*>(workspace), w, (hipStream_t)stream);
}

msa_status msa_workspace_status(const void* workspace, void* stream) {
  clear_error();
  const char* base = static_cast<const char*>(workspace);
  if (!base) {  // msa_decode_static's scratch on the current device
    char* ws = nullptr;
    msa_status st = static_scratch(&ws);
    if (st != MSA_OK) return st;
    base = ws;
  }
  if (!aligned(base, kAlign)) return fail(MSA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  uint32_t word = 0;
  hipStream_t hs = (hipStream_t)stream;
  msa_status st = hip_status(hipMemcpyAsync(&word, base, sizeof word, hipMemcpyDeviceToHost, hs),
                             "status read");
  if (st != MSA_OK) return st;
  st = hip_status(hipStreamSynchronize(hs), "status read");
  if (st != MSA_OK) return st;
  if (word != 0)
    return fail(MSA_ERR_DEVICE_WAIT,
                "a split-K merge gave up waiting for partial states; outputs of that call are "
                "NaN and the workspace must be zero-filled again before reuse");
  return MSA_OK;
}

void msa_set_merge_spin_limit(int32_t polls) { msa::set_merge_spin_limit(polls); }

msa_status msa_cache_write(const msa_problem* p, int32_t num_tokens, const int32_t* token_seq,
                           const int32_t* token_pos, const void* k_new, const void* v_new,
                           const void* ik_new, const int32_t* block_table, void* kv_data,
                           void* kv_scales, void* ik_data, void* ik_scales, void* stream) {
  msa_status st = msa_check_problem(p, kOpCacheWrite);
  if (st != MSA_OK) return st;
  if (num_tokens < 0) return fail(MSA_ERR_INVALID_ARGUMENT, "num_tokens < 0");
  if (num_tokens > 65535)
    return fail(MSA_ERR_UNSUPPORTED, "more than 65535 tokens in one call");
  if (num_tokens == 0) return MSA_OK;
  REQUIRE(token_seq, 4);
  REQUIRE(token_pos, 4);
  REQUIRE(k_new, 4);
  REQUIRE(v_new, 4);
  REQUIRE(ik_new, 4);
  REQUIRE(block_table, 4);
  REQUIRE(kv_data, 16);
  REQUIRE(ik_data, 16);
  if (p->kv_dtype == MSA_DTYPE_NVFP4) REQUIRE(kv_scales, 16);
  if (p->index_k_dtype == MSA_DTYPE_NVFP4) REQUIRE(ik_scales, 16);
  if (p->num_seqs == 0) return MSA_OK;
  const msa::Shape s = shape_of(p);
  return hip_status(msa::launch_cache_write(s, num_tokens, token_seq, token_pos, k_new, v_new,
                                            ik_new, block_table, kv_data, kv_scales, ik_data,
                                            ik_scales, (hipStream_t)stream),
                    "cache write launch");
}

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported problem";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MSA_ERR_HIP: return "HIP error";
    case MSA_ERR_DEVICE_WAIT: return "a device-side wait gave up";
    default: return "unknown status";
  }
}

const char* msa_last_error(void) { return g_err; }

}  // extern "C"
