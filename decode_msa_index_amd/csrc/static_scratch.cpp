// static_scratch.cpp -- msa_decode_static: the decode step for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).  Its scratch -- the split-K
// partial states, the status header and the pooled scores that msa_decode
// keeps in the caller's workspace -- lives in a file-scope device array of
// MSA_STATIC_SCRATCH_BYTES, one copy per GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "api_internal.hpp"

// In host code this name is only a host-side stand-in: kernels, fills and
// copies get the device address of the current GPU's copy, which
// hipGetSymbolAddress returns (looked up once per device, with that device
// current).
static __device__ __align__(256) unsigned char scratch[MSA_STATIC_SCRATCH_BYTES];

namespace msa_api {

namespace {
std::mutex g_mu;
std::vector<char*> g_ptr;  // per device id; nullptr until looked up
}  // namespace

msa_status static_scratch(char** out) {
  int dev = 0;
  msa_status st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != MSA_OK) return st;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((size_t)dev >= g_ptr.size()) g_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_ptr[(size_t)dev]) {
    void* ptr = nullptr;
    st = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)),
                    "hipGetSymbolAddress(scratch)");
    if (st != MSA_OK) return st;
    if (!ptr) return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_ptr[(size_t)dev] = static_cast<char*>(ptr);
  }
  *out = g_ptr[(size_t)dev];
  return MSA_OK;
}

}  // namespace msa_api

using namespace msa_api;

extern "C" msa_status msa_decode_static(const msa_problem* p, const void* index_q,
                                        const void* ik_data, const void* ik_scales, const void* q,
                                        const void* kv_data, const void* kv_scales,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const int32_t* q_pos, float* block_scores,
                                        int32_t* topk_idx, void* out, float* lse, void* stream) {
  msa_status st = check_decode_args(p, index_q, ik_data, ik_scales, q, kv_data, kv_scales,
                                    block_table, seq_lens, q_pos, block_scores, topk_idx, out,
                                    lse);
  if (st != MSA_OK) return st;
  const WsLayout w = ws_layout(p, kOpDecode);
  if (w.total > (size_t)MSA_STATIC_SCRATCH_BYTES)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "the problem needs %zu bytes of scratch, more than the %zu that "
                "msa_decode_static holds (pass block_scores, or call msa_decode with a "
                "workspace)",
                w.total, (size_t)MSA_STATIC_SCRATCH_BYTES);
  if (p->num_seqs == 0) return MSA_OK;
  char* ws = nullptr;
  st = static_scratch(&ws);
  if (st != MSA_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  // the array keeps the last call's contents (possibly a call that gave up
  // waiting): the part this call's kernels need zero -- the status header
  // and the split zone -- is cleared first, with a fill kernel rather than a
  // memset node
  const size_t zero_bytes = std::min(w.total, msa::kStatusBytes + msa::kSplitZoneBytes);
  st = hip_status(msa::launch_zero_fill(ws, zero_bytes, hs), "scratch clear launch");
  if (st != MSA_OK) return st;
  return decode_impl(p, index_q, ik_data, ik_scales, q, kv_data, kv_scales, block_table,
                     seq_lens, q_pos, block_scores, topk_idx, out, lse, ws, w, hs);
}
