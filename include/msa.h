/*
 * msa.h -- C ABI of the MI355X (gfx950) MiniMax Sparse Attention decode path.
 *
 * The method (vLLM blog "Day-0 support for MiniMax-M3.1-Flash", section "MSA
 * primer"): the KV cache is split into 128-token blocks; a lightning indexer
 * scores every cached key with one index query per GQA group against a single
 * shared index-key head; the token scores are max-pooled to one score per
 * block; exact attention then runs over the top-k (16) blocks only, with the
 * most recent block always kept, so a query sees at most k*128 keys.
 *
 * Four calls follow those steps:
 *   msa_index_scores   scores + per-block max-pool          (indexer)
 *   msa_block_topk     top-k blocks, recent block forced     (selection)
 *                      (and optional leading / trailing blocks)
 *   msa_sparse_attend  exact GQA attention over the blocks   (main attention)
 *   msa_decode         the three in one call
 * msa_decode's scores, selection, outputs and lse are bitwise those of the
 * three-call chain (both attend the selected blocks in ascending order with
 * the same launch shape, or both take the key-block path of
 * msa_sparse_attend).  A fifth call writes new tokens into the caches the
 * others read:
 *   msa_cache_write    quantise new K / V / index keys into their slots
 *
 * ---------------------------------------------------------------------------
 * Conventions
 * ---------------------------------------------------------------------------
 * All data pointers are DEVICE pointers owned by the caller; the library
 * allocates and frees nothing and keeps no state between calls (apart from
 * the test hook msa_set_merge_spin_limit).  Every call
 * validates its arguments on the host, synchronously, before anything is
 * launched, then enqueues its kernels on `stream` (a hipStream_t; NULL is the
 * default stream) and returns without waiting.  Device-side data (block-table
 * entries, sequence lengths, positions) are not read on the host; the kernels
 * bound every access by them instead:
 *   - a row sees keys t <= min(q_pos[r], seq_lens[b] - 1, MB*BS - 1) (without
 *     q_pos: t <= seq_lens[b] - 1 within the same reach);
 *   - a row that sees no key (seq_len 0, or q_pos < 0) gets -inf scores, an
 *     all -1 selection, a zero output and lse -inf;
 *   - block_table[b][j] is read only for the blocks a row sees; an entry
 *     outside [0, num_phys_blocks) is treated as an empty block (score -inf,
 *     no attention contribution), never dereferenced.
 * Sizes of the device buffers themselves are the caller's responsibility:
 * every array must have the extent given below.
 *
 * Shapes (B = num_seqs, R = rows_per_seq, G = num_kv_groups, H = num_q_heads,
 * D = head_dim, Di = index_dim, BS = block_size, P = num_phys_blocks,
 * MB = max_blocks_per_seq, K = top_k):
 *   index_q      [B*R][G][Di]        bf16 or f32          16-byte aligned
 *   q            [B*R][H][D]         bf16 or f32; head h uses group h/(H/G)
 *   index keys   fp8/f32: [P][BS][Di]
 *                nvfp4:   data [P][BS][Di/2] (even element in the low nibble)
 *                         scales [P][BS][Di/16] e4m3
 *   K/V cache    fp8/f32: [P][2][G][BS*D]; plane 0 = K stored [t][d],
 *                         plane 1 = V stored transposed [d][t]
 *                nvfp4:   data [P][2][G][BS*D/2]: K [t][d/2] (even d low),
 *                         V [d][t/2] (even t low);
 *                         scales [P][2][G][BS*D/16]: K [t][d/16], V [d/16][t]
 *   block_table  int32 [B][MB]       logical block -> physical block; one table
 *                                    serves the K/V and the index-key pools
 *   seq_lens     int32 [B]           cached tokens incl. the new one
 *   q_pos        int32 [B*R] or NULL position of each query row; keys t <= pos
 *                                    are visible.  NULL: R must be 1 and
 *                                    pos = seq_len - 1 (plain decode)
 *   block_scores f32 [B*R][G][MB]    pooled scores, -inf past the row's block
 *   topk_idx     int32 [B*R][G][K]   ascending logical block ids, -1 padded
 *   out          [B*R][H][D]         bf16 or f32          16-byte aligned
 *   lse          f32 [B*R][H] or NULL natural-log softmax denominator
 *
 * Number formats: bf16; OCP FP8 e4m3fn; NVFP4 = E2M1 values, one e4m3 scale
 * per 16 elements and a per-tensor fp32 scale passed as the *_scale field
 * (a dequantisation multiplier).  FP8 caches carry a per-tensor descale the
 * same way (k_scale, v_scale, index_k_scale).
 *
 * Status: every call returns an msa_status.  On failure nothing has been
 * enqueued (INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL) or a launch
 * failed (HIP); msa_last_error() then gives a thread-local message.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, inconsistent sizes */
  MSA_ERR_UNSUPPORTED = 2,      /* a shape or dtype combination not built */
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,
  MSA_ERR_HIP = 4,              /* a HIP launch or runtime call failed */
  MSA_ERR_DEVICE_WAIT = 5       /* msa_workspace_status: a split-K merge gave up
                                   waiting (see msa_workspace_bytes) */
} msa_status;

typedef enum {
  MSA_DTYPE_F32 = 0,
  MSA_DTYPE_BF16 = 1,
  MSA_DTYPE_FP8_E4M3 = 2,
  MSA_DTYPE_NVFP4 = 3
} msa_dtype;

/* Problem description, read on the host during the call only.  Zero-
 * initialise it (msa_problem p = {0};) and set the fields: the forced-block
 * counts at the end then default to 0. */
typedef struct msa_problem {
  int32_t num_seqs;           /* B >= 0 (0: nothing to do) */
  int32_t rows_per_seq;       /* R >= 1 query rows per sequence */
  int32_t num_q_heads;        /* H; H/G must be in [1, 16] */
  int32_t num_kv_groups;      /* G: KV heads = index heads; 1..8 */
  int32_t head_dim;           /* D: 128 */
  int32_t index_dim;          /* Di: 128 */
  int32_t block_size;         /* BS: 128 */
  int32_t top_k;              /* K: 1..32 blocks kept, recent included */
  int32_t max_blocks_per_seq; /* MB >= 1: block-table row stride */
  int32_t num_phys_blocks;    /* P >= 1 */
  int32_t q_dtype;            /* msa_dtype of q: BF16 or F32 */
  int32_t index_q_dtype;      /* msa_dtype of index_q: BF16 or F32 */
  int32_t kv_dtype;           /* msa_dtype of the K/V cache: FP8_E4M3, NVFP4, F32 */
  int32_t index_k_dtype;      /* msa_dtype of the index keys: FP8_E4M3, NVFP4, F32 */
  int32_t out_dtype;          /* msa_dtype of out: BF16 or F32 */
  float sm_scale;             /* attention logit multiplier (> 0), usually D^-0.5 */
  float index_scale;          /* index score multiplier (> 0), usually Di^-0.5 */
  float k_scale;              /* K dequant multiplier (> 0) */
  float v_scale;              /* V dequant multiplier */
  float index_k_scale;        /* index-key dequant multiplier (> 0) */
  int32_t init_blocks;        /* >= 0: leading blocks 0..init_blocks-1 always kept */
  int32_t local_blocks;       /* >= 0: the last max(local_blocks, 1) visible blocks
                                 always kept (0 and 1: the recent block alone);
                                 init_blocks + max(local_blocks, 1) <= top_k */
  int32_t share_seqs;         /* 0..64; 0 and 1: off.  n > 1: the sequences form
                                 consecutive share groups of n (the last may be
                                 shorter) whose block tables may point at the same
                                 physical blocks, e.g. requests with a common
                                 prefix.  The index scan then reads each distinct
                                 physical block of a logical block once for up to
                                 64 / num_kv_groups sequences of a group (pages
                                 dequantised once for the requests sharing them:
                                 blog "Day-0 support for MiniMax-M3.1-Flash",
                                 section "AMD NVFP4 MSA kernels").  A hint only:
                                 results are identical for any tables, nothing is
                                 assumed about them.  Needs rows_per_seq == 1;
                                 ignored for f32 index keys. */
} msa_problem;

/*
 * Host-side validation of a problem for one of the calls (op: 0 index
 * scores, 1 top-k, 2 sparse attend, 3 decode, 4 cache write).  Pure host
 * code; performs no HIP call.  Every entry point runs it first.
 */
msa_status msa_check_problem(const msa_problem* p, int32_t op);

/*
 * Workspace bytes a call needs for problem p (op as for msa_check_problem):
 *   - msa_sparse_attend: room for the split-K partial states when a (row,
 *     group) is split over several workgroups (0 when it is not); for a
 *     chunk of 640 or more rows per sequence over an FP8 or NVFP4 cache, the
 *     zone described below (which that path leaves alone) followed by the
 *     key-block path's buffers (see msa_sparse_attend): about 4.3 KB per
 *     (row, group, top-k slot), 1.1 GB for 4,096 rows at G = 4, top-16;
 *   - msa_decode: msa_sparse_attend's part, or at least the status header
 *     and the whole zone described below (256 + 4,259,840 bytes), then
 *     B*R*G*MB words for the pooled scores: they lie past the zone, every
 *     call writes all of them before reading them, and they are not cleared;
 *   - the other calls: 0.
 * Every region is rounded up to 256 bytes, and a workspace that holds
 * partial states starts with a 256-byte status header.  The workspace is
 * caller-owned device memory, 256-byte aligned.  msa_decode requires its
 * first 256 + 4,259,840 bytes (all of it, if smaller) to be zero-filled
 * before its first use (e.g. hipMemset once after allocation): the status
 * header and the zone where the split-K partial states of any problem shape
 * live -- the workgroups of the attention kernel hand partial states to
 * each other through it, and a word still zero means "not yet written".
 * Every msa_decode and msa_sparse_attend call leaves that part zero-filled
 * again, so one zero fill serves any sequence of calls and problem shapes;
 * past it a call may leave its scratch (msa_decode's pooled scores, the
 * key-block path's lists and partials).  msa_sparse_attend
 * itself needs no initialisation (it clears what it uses).  Calls that
 * share a workspace must not overlap.  A call whose size is 0 accepts a
 * NULL workspace.
 *
 * Failure mode: the workgroup that merges a (row, group)'s partial states
 * waits for them with a bounded poll (about a second).  Should it ever give
 * up, that (row, group)'s out and lse become NaN, the call has already
 * returned MSA_OK, and the workspace is marked in its status header instead
 * of being cleared (a partial state could still land after a clearing).
 * msa_workspace_status reads the mark; later msa_decode calls on a marked
 * workspace give NaN for every split (row, group) until the caller
 * zero-fills it again.  msa_sparse_attend, and msa_decode calls that run the
 * three calls' kernels (block tables over 8064 blocks per row), clear the
 * header and the zone at the start of any call that splits a (row, group)
 * over workgroups, like a caller's zero fill.  The key-block path (chunks of
 * 640 or more rows per sequence) uses neither and leaves both as they are,
 * a mark included.
 */
msa_status msa_workspace_bytes(const msa_problem* p, int32_t op, size_t* bytes);

/*
 * Indexer scores + block max-pool (blog, "MSA primer"; API reference of
 * MiniMaxM3SparseAttention: one index head per KV head, scale Di^-0.5,
 * sparse_score_type "max").  For every row r, group g and logical block j:
 *   score(t) = index_scale * index_k_scale * sum_d index_q[r][g][d] * key(t, d)
 *   block_scores[r][g][j] = max over visible t in block j of score(t)
 * and -inf for blocks past the row's last visible block.  fp32 arithmetic on
 * exactly dequantised operands.  ik_scales is required for NVFP4 index keys
 * and ignored otherwise.
 */
msa_status msa_index_scores(const msa_problem* p, const void* index_q, const void* ik_data,
                            const void* ik_scales, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* q_pos,
                            float* block_scores, void* stream);

/*
 * Block selection (blog, "MSA primer": top 16 blocks, most recent block
 * always kept).  For row r with last visible block rb = pos / BS: if
 * rb + 1 <= K all blocks 0..rb are kept.  Otherwise the forced blocks are
 * kept -- 0 .. init_blocks-1 and the last L = max(local_blocks, 1) blocks
 * rb-L+1 .. rb (the indexer's init_blocks / local_blocks, which the API
 * reference of MiniMaxM3SparseAttention's constructor fills from
 * sparse_init_block / sparse_local_block; read as blocks always kept inside
 * the k) -- plus the K - init_blocks - L best of the
 * free blocks init_blocks .. rb-L by (block_scores descending, block index
 * ascending).  With init_blocks = local_blocks = 0 that is rb plus the K-1
 * best of 0..rb-1.  Output ascending, -1 padded.  Deterministic: ties go to
 * the lower block index.  block_scores entries must not be NaN.
 */
msa_status msa_block_topk(const msa_problem* p, const float* block_scores,
                          const int32_t* seq_lens, const int32_t* q_pos, int32_t* topk_idx,
                          void* stream);

/*
 * Exact sparse GQA attention over the selected blocks (blog, "MSA primer",
 * Figure 1: every query head of a group attends exactly the group's
 * blocks).  For head h of group g and visible tokens t of the selected
 * blocks: out = sum_t softmax_t(sm_scale * k_scale * q.k_t) * v_scale * v_t,
 * with fp32 softmax state, split over the selected blocks (across the waves
 * of a workgroup and, for small batches, across workgroups, one of which
 * merges the others' partial states).  A chunk of 640 or more rows per
 * sequence over an FP8 or NVFP4 cache (chunked prefill) is grouped by key
 * block instead (API reference, MiniMaxM3Model: the top-k buffer inverted by
 * build_k2q_csr): each selected block is read and dequantised once per up to
 * 64 rows that selected it, each (row, group, block) leaves a partial whose
 * output is rounded to f16, and each row's partials are merged in selection
 * order with fp32 weights; out and lse then differ from a per-row gather by
 * that rounding (relative 2^-11 of each partial).  topk_idx: the first
 * min(top_k, last visible block + 1) entries of a row are read; an entry
 * outside [0, last visible block] contributes nothing (msa_block_topk never
 * writes one).  kv_scales is required for NVFP4 and ignored otherwise.  lse
 * may be NULL.  workspace: msa_workspace_bytes(p, 2) bytes (may be NULL when
 * that is 0).
 */
msa_status msa_sparse_attend(const msa_problem* p, const void* q, const void* kv_data,
                             const void* kv_scales, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* q_pos,
                             const int32_t* topk_idx, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole decode step (blog, "MSA primer"): msa_index_scores ->
 * msa_block_topk -> msa_sparse_attend; scores, selection, out and lse are
 * bitwise the three calls'.  For FP8 or NVFP4 caches and block tables of up
 * to 8064 blocks per row (about a million tokens) it is two kernels, the
 * scan and then selection + attention in one; chunks of 640 or more rows
 * per sequence, longer tables and fp32 caches run the three calls' kernels
 * in turn.
 * topk_idx receives the selection; block_scores (nullable) receives the
 * pooled scores.  workspace: msa_workspace_bytes(p, 3) bytes, its first
 * 256 + 4,259,840 bytes zero-filled before its first use and left
 * zero-filled (see msa_workspace_bytes).
 */
msa_status msa_decode(const msa_problem* p, const void* index_q, const void* ik_data,
                      const void* ik_scales, const void* q, const void* kv_data,
                      const void* kv_scales, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* q_pos, float* block_scores,
                      int32_t* topk_idx, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Cache write, the insert half of a decode step (blog, "MSA primer": FP8 index
 * keys of 128 B per token; the NVFP4 kernels section: E2M1 values with one
 * e4m3 scale per 16 elements and a per-tensor scale).  New token i belongs to
 * sequence token_seq[i] at position token_pos[i]; its slot is logical block
 * token_pos[i] / BS of that sequence (through block_table), row
 * token_pos[i] % BS.  Its K and V for every group and its index key are
 * quantised into kv_data / kv_scales and ik_data / ik_scales, in the layouts
 * the other calls read, so that their dequantisation gives the values back
 * to the format's precision.  Every step is one correctly rounded binary32
 * operation, with scale = k_scale, v_scale or index_k_scale:
 *   F32  : x / scale
 *   FP8  : e4m3(x / scale), round to nearest even, saturating at +-448
 *   NVFP4: per 16 consecutive elements of a token (K and index keys: 16
 *          dims of the row; V: 16 dims of the token's column),
 *          s = e4m3(amax / (6 * scale)); element e2m1(x / (e4m3(s) * scale)),
 *          nearest even, saturating at +-6; all 0 when s is 0.
 * Inputs: k_new, v_new [num_tokens][G][D] in q_dtype, ik_new
 * [num_tokens][Di] in index_q_dtype, all finite.  The other tokens' slots
 * are not touched (V's NVFP4 nibbles shared with a neighbour token are
 * updated atomically).  Tokens whose sequence, position or table entry is
 * out of range are skipped.  Two new tokens must not map to the same slot.
 * num_tokens <= 65535 per call.  Format pairs as for msa_decode.
 */
msa_status msa_cache_write(const msa_problem* p, int32_t num_tokens, const int32_t* token_seq,
                           const int32_t* token_pos, const void* k_new, const void* v_new,
                           const void* ik_new, const int32_t* block_table, void* kv_data,
                           void* kv_scales, void* ik_data, void* ik_scales, void* stream);

/*
 * msa_decode without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, semantics and results as msa_decode,
 * minus the workspace: its scratch is a device array of
 * MSA_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  A problem whose msa_workspace_bytes(p, 3) exceeds that is
 * rejected with MSA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued
 * (passing block_scores does not shrink the need: the size is that of the
 * decode workspace).  The call allocates nothing: it clears the scratch
 * region it needs with a fill kernel, then enqueues the decode.  Every call
 * on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 * msa_workspace_status(NULL, stream) reads the array's status header.
 */
#define MSA_STATIC_SCRATCH_BYTES (16u << 20)
msa_status msa_decode_static(const msa_problem* p, const void* index_q, const void* ik_data,
                             const void* ik_scales, const void* q, const void* kv_data,
                             const void* kv_scales, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* q_pos, float* block_scores,
                             int32_t* topk_idx, void* out, float* lse, void* stream);

/*
 * Status of a workspace after the calls enqueued on `stream` so far: waits
 * for the stream, reads the status header of `workspace` (a decode or attend
 * workspace of at least 256 bytes; NULL: msa_decode_static's scratch on the
 * current device) and returns MSA_ERR_DEVICE_WAIT if a
 * split-K merge gave up waiting on it (see msa_workspace_bytes), MSA_OK
 * otherwise.  Synchronous: not for use inside a captured graph.
 */
msa_status msa_workspace_status(const void* workspace, void* stream);

/*
 * Test hook for the failure path above: polls of one batch of partial states
 * before a merging workgroup gives up, for launches enqueued after the call
 * (default 2^20; a negative value makes every merge give up at once, so that
 * the NaN outputs and the status mark can be checked while every kernel
 * still runs to its normal end).  Process-wide; not for production use.
 */
void msa_set_merge_spin_limit(int32_t polls);

/* Static description of a status code. */
const char* msa_status_string(msa_status s);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* msa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
