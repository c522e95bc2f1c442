/*
 * msa_oracle.c -- plain CPU oracle of the MSA decode path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path.  It shares no
 * code with the HIP library.  See msa_oracle.h for the layouts.
 *
 * Each function below is the definition written out, one element at a time,
 * in double precision.  Threads only split independent (row, group) units;
 * the result does not depend on the thread count.
 */
#include "msa_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* Element formats                                                          */
/* ------------------------------------------------------------------------ */

/* OCP FP8 e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent field 0 is subnormal m/8 * 2^-6.
 * The KV caches and index keys are e4m3 (vLLM blog, "MSA primer": 128 B per
 * token of FP8 index key; PR #45744 report: e4m3 allowed, e5m2 excluded). */
double msa_oracle_e4m3(uint8_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* E2M1 (FP4): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
 * subnormal m * 0.5.  Magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.  NVFP4 = E2M1
 * values with one e4m3 scale per 16 elements and a per-tensor scale (vLLM
 * blog, "AMD NVFP4 MSA kernels": 256 possible e4m3 scales x 8 E2M1
 * magnitudes). */
double msa_oracle_e2m1(uint8_t nibble) {
  int s = (nibble >> 3) & 1;
  int e = (nibble >> 1) & 3;
  int m = nibble & 1;
  double v;
  if (e == 0)
    v = 0.5 * (double)m;
  else
    v = ldexp(1.0 + 0.5 * (double)m, e - 1);
  return s ? -v : v;
}

/* Encoders, by their definition: the code whose value is nearest to x, a
 * tie going to the code whose last bit is 0 (round to nearest, ties to
 * even); magnitudes beyond the largest finite value take it (saturation);
 * the sign is kept, so negative values that round to zero give -0.  x must
 * not be NaN.  A search over the finite codes, with no bit tricks. */
uint8_t msa_oracle_encode_e4m3(double x) {
  int neg = signbit(x) != 0;
  double a = fabs(x);
  int best = 0x7E;  /* 448: the answer for +inf and every a >= 448 */
  double best_err = INFINITY;
  if (!isinf(a)) {
    for (int c = 0; c <= 0x7E; ++c) {  /* 0x7F is NaN */
      double err = fabs(msa_oracle_e4m3((uint8_t)c) - a);
      if (err < best_err || (err == best_err && (c & 1) == 0)) {
        best = c;
        best_err = err;
      }
    }
  }
  return (uint8_t)(best | (neg ? 0x80 : 0));
}

uint8_t msa_oracle_encode_e2m1(double x) {
  int neg = signbit(x) != 0;
  double a = fabs(x);
  int best = 7;  /* 6.0 */
  double best_err = INFINITY;
  if (!isinf(a)) {
    for (int c = 0; c <= 7; ++c) {
      double err = fabs(msa_oracle_e2m1((uint8_t)c) - a);
      if (err < best_err || (err == best_err && (c & 1) == 0)) {
        best = c;
        best_err = err;
      }
    }
  }
  return (uint8_t)(best | (neg ? 8 : 0));
}

/* bfloat16 is the upper half of an IEEE binary32. */
double msa_oracle_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double read_plain(int dtype, const void* base, size_t idx) {
  switch (dtype) {
    case MSA_OR_F32: return (double)((const float*)base)[idx];
    case MSA_OR_BF16: return msa_oracle_bf16(((const uint16_t*)base)[idx]);
    case MSA_OR_FP8: return msa_oracle_e4m3(((const uint8_t*)base)[idx]);
    default: return NAN;
  }
}

/* NVFP4 element: data byte idx/2 (even index in the low nibble) times the
 * e4m3 scale that covers it. */
static double read_nvfp4(const void* data, size_t elem, const void* scales,
                         size_t scale_idx) {
  uint8_t byte = ((const uint8_t*)data)[elem / 2];
  uint8_t nib = (elem & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
  return msa_oracle_e4m3(((const uint8_t*)scales)[scale_idx]) *
         msa_oracle_e2m1(nib);
}

/* Index key element (physical block p, slot t, dim d), without the tensor
 * scale. */
static double index_key(const msa_oracle_problem* p, const void* data,
                        const void* scales, int64_t pb, int t, int d) {
  size_t row = (size_t)pb * (size_t)p->block_size + (size_t)t;
  if (p->index_k_dtype == MSA_OR_NVFP4)
    return read_nvfp4(data, row * (size_t)p->index_dim + (size_t)d, scales,
                      row * (size_t)(p->index_dim / 16) + (size_t)(d / 16));
  return read_plain(p->index_k_dtype, data, row * (size_t)p->index_dim + (size_t)d);
}

/* K or V element (physical block pb, group g, slot t, dim d), without the
 * tensor scale.  kv = 0 reads K ([t][d]); kv = 1 reads V, stored [d][t]. */
static double kv_elem(const msa_oracle_problem* p, const void* data,
                      const void* scales, int64_t pb, int kv, int g, int t, int d) {
  size_t plane = ((size_t)pb * 2 + (size_t)kv) * (size_t)p->num_groups + (size_t)g;
  size_t per = (size_t)p->block_size * (size_t)p->head_dim;
  size_t inner = kv == 0 ? (size_t)t * (size_t)p->head_dim + (size_t)d
                         : (size_t)d * (size_t)p->block_size + (size_t)t;
  if (p->kv_dtype == MSA_OR_NVFP4) {
    size_t sidx = kv == 0 ? (size_t)t * (size_t)(p->head_dim / 16) + (size_t)(d / 16)
                          : (size_t)(d / 16) * (size_t)p->block_size + (size_t)t;
    return read_nvfp4(data, plane * per + inner, scales, plane * (per / 16) + sidx);
  }
  return read_plain(p->kv_dtype, data, plane * per + inner);
}

/* ------------------------------------------------------------------------ */
/* Rows, positions, validity                                                */
/* ------------------------------------------------------------------------ */

static int check_problem(const msa_oracle_problem* p) {
  if (!p) return -1;
  if (p->num_seqs < 0 || p->rows_per_seq < 1 || p->num_groups < 1 ||
      p->num_q_heads < p->num_groups || p->num_q_heads % p->num_groups ||
      p->head_dim < 16 || p->head_dim % 16 || p->index_dim < 16 ||
      p->index_dim % 16 || p->block_size < 2 || p->block_size % 2 ||
      p->top_k < 1 || p->max_blocks < 1 || p->num_phys_blocks < 1 ||
      p->init_blocks < 0 || p->local_blocks < 0 ||
      p->init_blocks + (p->local_blocks > 1 ? p->local_blocks : 1) > p->top_k)
    return -1;
  return 0;
}

/* Last visible key of the query row: keys t <= pos and t < seq_len are
 * visible, and only keys the block table reaches (t < max_blocks * block_size:
 * a row cannot see a block it has no table entry for).  Decode rows see the
 * whole cache, including the token just inserted.  A negative result means
 * the row sees no key at all.  (The pages say nothing of a sequence longer
 * than its table; this is the reading the library's header documents.) */
static int64_t row_pos(const msa_oracle_problem* p, const int32_t* seq_lens,
                       const int32_t* q_pos, int64_t row) {
  int64_t b = row / p->rows_per_seq;
  int64_t reach = (int64_t)p->max_blocks * p->block_size;
  int64_t last = (int64_t)seq_lens[b] < reach ? (int64_t)seq_lens[b] : reach;
  last -= 1;
  if (q_pos && (int64_t)q_pos[row] < last) return q_pos[row];
  return last;
}

/* Physical block of logical block j of sequence b, or -1 when the table
 * entry lies outside the pool [0, num_phys_blocks): such a block holds no
 * key (pooled score -inf, nothing to attend).  The pages are silent on
 * malformed tables; this is the reading the library's header documents. */
static int64_t phys_block(const msa_oracle_problem* p, const int32_t* block_table,
                          int64_t b, int64_t j) {
  int64_t pb = block_table[b * (int64_t)p->max_blocks + j];
  return (pb < 0 || pb >= p->num_phys_blocks) ? -1 : pb;
}

/* ------------------------------------------------------------------------ */
/* Thread fan-out over independent (row, group) units                       */
/* ------------------------------------------------------------------------ */

typedef void (*unit_fn)(void* ctx, int64_t unit);
typedef struct {
  unit_fn fn;
  void* ctx;
  int64_t n_units;
  int nthreads;
  int tid;
} fan_arg;

static int g_threads_used = 1;

static void* fan_worker(void* a_) {
  fan_arg* a = (fan_arg*)a_;
  for (int64_t u = a->tid; u < a->n_units; u += a->nthreads) a->fn(a->ctx, u);
  return NULL;
}

static void fan_out(int requested, int64_t n_units, unit_fn fn, void* ctx) {
  int nt = requested > 0 ? requested : (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nt < 1) nt = 1;
  if (nt > 256) nt = 256;
  if ((int64_t)nt > n_units) nt = n_units > 0 ? (int)n_units : 1;
  g_threads_used = nt;
  pthread_t th[256];
  fan_arg args[256];
  for (int i = 0; i < nt; ++i) {
    args[i].fn = fn;
    args[i].ctx = ctx;
    args[i].n_units = n_units;
    args[i].nthreads = nt;
    args[i].tid = i;
  }
  if (nt == 1) {
    fan_worker(&args[0]);
    return;
  }
  for (int i = 0; i < nt; ++i) pthread_create(&th[i], NULL, fan_worker, &args[i]);
  for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
}

int msa_oracle_threads_used(void) { return g_threads_used; }

/* ------------------------------------------------------------------------ */
/* Step 1+2: index scores and block max-pool                                */
/* ------------------------------------------------------------------------ */

/* Score of the token in slot `slot` of physical block pb for (row, group):
 * the dot product of the group's index query with the shared index key,
 * times the score scale, in double, then rounded once to binary32.  One index query per GQA group, one index-key
 * head shared by all groups (vLLM blog, "MSA primer"; API reference of
 * MiniMaxM3SparseAttention: the indexer is built with scale = head_dim^-0.5
 * and num_index_heads = num_kv_heads). */
static float token_score(const msa_oracle_problem* p, const void* index_q,
                         const void* ik_data, const void* ik_scales, int64_t pb,
                         int64_t row, int g, int slot) {
  size_t qoff = ((size_t)row * (size_t)p->num_groups + (size_t)g) * (size_t)p->index_dim;
  double dot = 0.0;
  for (int d = 0; d < p->index_dim; ++d) {
    double qd = read_plain(p->index_q_dtype, index_q, qoff + (size_t)d);
    double kd = index_key(p, ik_data, ik_scales, pb, slot, d);
    dot += qd * kd;
  }
  return (float)(p->index_scale * p->index_k_scale * dot);
}

typedef struct {
  const msa_oracle_problem* p;
  const void *index_q, *ik_data, *ik_scales;
  const int32_t *block_table, *seq_lens, *q_pos;
  float* scores;
} score_ctx;

/* Max-pool: the score of logical block j is the largest token score over
 * the block's visible tokens (sparse_score_type "max" in the API reference
 * of MiniMaxM3SparseAttention.__init__).  Blocks past the row's last visible
 * block, and blocks whose table entry is outside the pool, get -inf. */
static void score_unit(void* c_, int64_t unit) {
  score_ctx* c = (score_ctx*)c_;
  const msa_oracle_problem* p = c->p;
  int64_t row = unit / p->num_groups;
  int g = (int)(unit % p->num_groups);
  int64_t pos = row_pos(p, c->seq_lens, c->q_pos, row);
  float* out = c->scores + (size_t)unit * (size_t)p->max_blocks;
  for (int64_t j = 0; j < p->max_blocks; ++j) {
    int64_t t0 = j * p->block_size;
    if (t0 > pos) {
      out[j] = -INFINITY;
      continue;
    }
    int64_t t1 = t0 + p->block_size - 1;
    if (t1 > pos) t1 = pos;
    int64_t pb = phys_block(p, c->block_table, row / p->rows_per_seq, j);
    float best = -INFINITY;  /* the max over no token: an empty block */
    for (int64_t t = t0; pb >= 0 && t <= t1; ++t) {
      float s = token_score(p, c->index_q, c->ik_data, c->ik_scales, pb, row, g,
                            (int)(t - t0));
      if (s > best) best = s;
    }
    out[j] = best;
  }
}

int msa_oracle_index_scores(const msa_oracle_problem* p, const void* index_q,
                            const void* ik_data, const void* ik_scales,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* q_pos, float* scores) {
  if (check_problem(p) || !index_q || !ik_data || !block_table || !seq_lens || !scores)
    return -1;
  if (p->index_k_dtype == MSA_OR_NVFP4 && !ik_scales) return -1;
  score_ctx c = {p, index_q, ik_data, ik_scales, block_table, seq_lens, q_pos, scores};
  int64_t units = (int64_t)p->num_seqs * p->rows_per_seq * p->num_groups;
  fan_out(p->num_threads, units, score_unit, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 3: block top-k, most recent block forced                            */
/* ------------------------------------------------------------------------ */

typedef struct {
  float s;
  int32_t j;
} cand;

/* Order: higher pooled score first; equal scores go to the lower logical
 * block index. */
static int cand_cmp(const void* a_, const void* b_) {
  const cand* a = (const cand*)a_;
  const cand* b = (const cand*)b_;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j > b->j) - (a->j < b->j);
}

static int int_cmp(const void* a_, const void* b_) {
  int32_t a = *(const int32_t*)a_, b = *(const int32_t*)b_;
  return (a > b) - (a < b);
}

typedef struct {
  const msa_oracle_problem* p;
  const float* scores;
  const int32_t *seq_lens, *q_pos;
  int32_t* topk;
} topk_ctx;

/* The top-k blocks with the most recent block always kept, so at most
 * top_k * block_size keys per query (vLLM blog, "MSA primer": top 16 blocks,
 * most recent block always kept, at most 2,048 keys).  The recent block is
 * the one holding the row's own position; it counts inside the k.
 *
 * The indexer also takes sparse_init_block and sparse_local_block (vLLM API
 * reference of vllm.models.minimax_m3.nvidia.model, the
 * MiniMaxM3SparseAttention constructor: passed on as init_blocks and
 * local_blocks, both 0 unless configured; nothing more is said of them).
 * Read here as blocks that are always kept besides the recent one, inside
 * the k like it: the first init_blocks blocks 0 .. init_blocks-1 and the
 * last max(local_blocks, 1) blocks of 0..recent (so local_blocks 0 and 1
 * both mean the recent block alone).  The k - (number forced) best of the
 * remaining blocks fill the rest, by score and then lower block index.
 * Output: ascending logical ids, then -1. */
static void topk_unit(void* c_, int64_t unit) {
  topk_ctx* c = (topk_ctx*)c_;
  const msa_oracle_problem* p = c->p;
  int64_t row = unit / p->num_groups;
  int64_t pos = row_pos(p, c->seq_lens, c->q_pos, row);
  const float* s = c->scores + (size_t)unit * (size_t)p->max_blocks;
  int32_t* out = c->topk + (size_t)unit * (size_t)p->top_k;
  if (pos < 0) { /* no visible key: nothing to select */
    for (int32_t i = 0; i < p->top_k; ++i) out[i] = -1;
    return;
  }
  int32_t recent = (int32_t)(pos / p->block_size);
  int32_t n_local = p->local_blocks > 1 ? p->local_blocks : 1;
  int32_t n_sel = 0;
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)p->top_k);
  if (recent + 1 <= p->top_k) {
    for (int32_t j = 0; j <= recent; ++j) sel[n_sel++] = j;
  } else {
    cand* cs = (cand*)malloc(sizeof(cand) * (size_t)(recent + 1));
    int32_t n_cand = 0;
    for (int32_t j = 0; j <= recent; ++j) {
      int forced = j < p->init_blocks || j > recent - n_local;
      if (forced) {
        sel[n_sel++] = j;
      } else {
        cs[n_cand].s = s[j];
        cs[n_cand].j = j;
        ++n_cand;
      }
    }
    qsort(cs, (size_t)n_cand, sizeof(cand), cand_cmp);
    for (int32_t i = 0; n_sel < p->top_k && i < n_cand; ++i) sel[n_sel++] = cs[i].j;
    free(cs);
    qsort(sel, (size_t)n_sel, sizeof(int32_t), int_cmp);
  }
  for (int32_t i = 0; i < p->top_k; ++i) out[i] = i < n_sel ? sel[i] : -1;
  free(sel);
}

int msa_oracle_block_topk(const msa_oracle_problem* p, const float* scores,
                          const int32_t* seq_lens, const int32_t* q_pos,
                          int32_t* topk) {
  if (check_problem(p) || !scores || !seq_lens || !topk) return -1;
  topk_ctx c = {p, scores, seq_lens, q_pos, topk};
  int64_t units = (int64_t)p->num_seqs * p->rows_per_seq * p->num_groups;
  fan_out(p->num_threads, units, topk_unit, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 4: exact GQA softmax attention over the selected blocks             */
/* ------------------------------------------------------------------------ */

typedef struct {
  const msa_oracle_problem* p;
  const void *q, *kv_data, *kv_scales;
  const int32_t *block_table, *seq_lens, *q_pos, *topk;
  double *out, *lse;
} attend_ctx;

/* Every query head of group g attends exactly the group's selected blocks
 * (vLLM blog, "MSA primer", Figure 1 caption); within them the attention is
 * the ordinary softmax(sm_scale * q.k) weighted sum of v over the visible
 * tokens (t <= pos).  sm_scale is head_dim^-0.5 in the API reference of
 * MiniMaxM3SparseAttention. */
static void attend_unit(void* c_, int64_t unit) {
  attend_ctx* c = (attend_ctx*)c_;
  const msa_oracle_problem* p = c->p;
  int64_t row = unit / p->num_groups;
  int g = (int)(unit % p->num_groups);
  int64_t b = row / p->rows_per_seq;
  int64_t pos = row_pos(p, c->seq_lens, c->q_pos, row);
  const int32_t* sel = c->topk + (size_t)unit * (size_t)p->top_k;
  int hpg = p->num_q_heads / p->num_groups;
  int D = p->head_dim;

  /* gather the visible tokens of the selected blocks */
  int64_t max_tok = (int64_t)p->top_k * p->block_size;
  int64_t* tok_pb = (int64_t*)malloc(sizeof(int64_t) * (size_t)max_tok);
  int* tok_slot = (int*)malloc(sizeof(int) * (size_t)max_tok);
  int64_t n = 0;
  for (int i = 0; i < p->top_k; ++i) {
    int32_t j = sel[i];
    if (j < 0) continue;
    int64_t pb = phys_block(p, c->block_table, b, j);
    if (pb < 0) continue; /* an entry outside the pool holds no key */
    for (int t = 0; t < p->block_size; ++t) {
      int64_t tok = (int64_t)j * p->block_size + t;
      if (tok > pos) break;
      tok_pb[n] = pb;
      tok_slot[n] = t;
      ++n;
    }
  }
  double* logit = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int hh = 0; hh < hpg; ++hh) {
    int h = g * hpg + hh;
    size_t qoff = ((size_t)row * (size_t)p->num_q_heads + (size_t)h) * (size_t)D;
    double* o = c->out + qoff;
    double mx = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += read_plain(p->q_dtype, c->q, qoff + (size_t)d) *
               (p->k_scale * kv_elem(p, c->kv_data, c->kv_scales, tok_pb[i], 0, g,
                                     tok_slot[i], d));
      logit[i] = p->sm_scale * dot;
      if (logit[i] > mx) mx = logit[i];
    }
    double den = 0.0;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      double w = exp(logit[i] - mx);
      den += w;
      for (int d = 0; d < D; ++d)
        o[d] += w * (p->v_scale * kv_elem(p, c->kv_data, c->kv_scales, tok_pb[i], 1,
                                          g, tok_slot[i], d));
    }
    for (int d = 0; d < D; ++d) o[d] = n > 0 ? o[d] / den : 0.0;
    if (c->lse)
      c->lse[(size_t)row * (size_t)p->num_q_heads + (size_t)h] =
          n > 0 ? mx + log(den) : -INFINITY;
  }
  free(logit);
  free(tok_pb);
  free(tok_slot);
}

int msa_oracle_sparse_attend(const msa_oracle_problem* p, const void* q,
                             const void* kv_data, const void* kv_scales,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* q_pos, const int32_t* topk,
                             double* out, double* lse) {
  if (check_problem(p) || !q || !kv_data || !block_table || !seq_lens || !topk || !out)
    return -1;
  if (p->kv_dtype == MSA_OR_NVFP4 && !kv_scales) return -1;
  attend_ctx c = {p, q, kv_data, kv_scales, block_table, seq_lens, q_pos, topk, out, lse};
  int64_t units = (int64_t)p->num_seqs * p->rows_per_seq * p->num_groups;
  fan_out(p->num_threads, units, attend_unit, &c);
  return 0;
}

int msa_oracle_decode(const msa_oracle_problem* p, const void* index_q,
                      const void* ik_data, const void* ik_scales, const void* q,
                      const void* kv_data, const void* kv_scales,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* q_pos, float* scores, int32_t* topk,
                      double* out, double* lse) {
  int rc = msa_oracle_index_scores(p, index_q, ik_data, ik_scales, block_table,
                                   seq_lens, q_pos, scores);
  if (rc) return rc;
  rc = msa_oracle_block_topk(p, scores, seq_lens, q_pos, topk);
  if (rc) return rc;
  return msa_oracle_sparse_attend(p, q, kv_data, kv_scales, block_table, seq_lens,
                                  q_pos, topk, out, lse);
}

/* ------------------------------------------------------------------------ */
/* Cache write: quantise new tokens into the paged caches                   */
/* ------------------------------------------------------------------------ */

/* binary32 rounding of a double: every step below is one correctly rounded
 * binary32 operation (a double result of an operation on binary32 operands,
 * rounded once to binary32, is the correctly rounded binary32 result). */
static double f32(double x) { return (double)(float)x; }

/* Stores the `n` values x[0..n) of one cache row (or column) in format
 * `dtype` with dequant multiplier `scale`: element i goes to code index
 * idx(i) of data; for NVFP4 the e4m3 scale of group i/16 goes to scale index
 * sidx(i/16).  Plain: code = round(x / scale) in the cache's format.  NVFP4
 * (the generator's quantiser, with the given tensor scale g = scale): per
 * group of 16, s = e4m3(amax / (6 g)); element q = e2m1(x / (e4m3value(s) g)),
 * 0 when the scale is 0. */
typedef size_t (*index_fn)(const void* ctx, int i);

static void store_row(int dtype, double scale, const double* x, int n, void* data, void* scales,
                      index_fn idx, index_fn sidx, const void* ctx) {
  double sc = f32(scale);
  if (dtype == MSA_OR_NVFP4) {
    for (int g0 = 0; g0 < n; g0 += 16) {
      double amax = 0.0;
      for (int i = g0; i < g0 + 16; ++i) amax = fmax(amax, fabs(x[i]));
      uint8_t s = msa_oracle_encode_e4m3(f32(amax / f32(6.0 * sc)));
      ((uint8_t*)scales)[sidx(ctx, g0 / 16)] = s;
      double sg = f32(msa_oracle_e4m3(s) * sc);
      for (int i = g0; i < g0 + 16; ++i) {
        uint8_t q = sg == 0.0 ? 0 : msa_oracle_encode_e2m1(f32(x[i] / sg));
        size_t e = idx(ctx, i);
        uint8_t* byte = (uint8_t*)data + e / 2;
        *byte = (e & 1) ? (uint8_t)((*byte & 0x0F) | (q << 4)) : (uint8_t)((*byte & 0xF0) | q);
      }
    }
    return;
  }
  for (int i = 0; i < n; ++i) {
    double v = f32(x[i] / sc);
    if (dtype == MSA_OR_FP8)
      ((uint8_t*)data)[idx(ctx, i)] = msa_oracle_encode_e4m3(v);
    else
      ((float*)data)[idx(ctx, i)] = (float)v;
  }
}

/* element index of a row: K / index keys are token-major ([t][d]), V is
 * stored transposed ([d][t]) */
typedef struct {
  size_t base, row_len;  /* element index of (t = 0, d = 0) of the plane; D or BS */
  int t, bs, transposed;
} row_ctx;

static size_t row_elem(const void* c_, int d) {
  const row_ctx* c = (const row_ctx*)c_;
  return c->transposed ? c->base + (size_t)d * (size_t)c->bs + (size_t)c->t
                       : c->base + (size_t)c->t * c->row_len + (size_t)d;
}
static size_t row_scale(const void* c_, int grp) {
  const row_ctx* c = (const row_ctx*)c_;
  return c->transposed ? c->base / 16 + (size_t)grp * (size_t)c->bs + (size_t)c->t
                       : c->base / 16 + (size_t)c->t * (c->row_len / 16) + (size_t)grp;
}

int msa_oracle_cache_write(const msa_oracle_problem* p, int32_t num_tokens,
                           const int32_t* token_seq, const int32_t* token_pos,
                           const void* k_new, const void* v_new, const void* ik_new,
                           const int32_t* block_table, void* kv_data, void* kv_scales,
                           void* ik_data, void* ik_scales) {
  if (check_problem(p) || num_tokens < 0) return -1;
  const int G = p->num_groups, D = p->head_dim, Di = p->index_dim, BS = p->block_size;
  double* x = (double*)malloc(sizeof(double) * (size_t)(D > Di ? D : Di));
  if (!x) return -1;
  for (int32_t i = 0; i < num_tokens; ++i) {
    int32_t b = token_seq[i], pos = token_pos[i];
    if (b < 0 || b >= p->num_seqs || pos < 0 || pos >= p->max_blocks * BS) continue;
    int32_t pb = block_table[(size_t)b * (size_t)p->max_blocks + (size_t)(pos / BS)];
    if (pb < 0 || pb >= p->num_phys_blocks) continue;
    int t = pos % BS;
    for (int kv = 0; kv < 2; ++kv) {
      const void* src = kv == 0 ? k_new : v_new;
      double scale = kv == 0 ? p->k_scale : p->v_scale;
      for (int g = 0; g < G; ++g) {
        for (int d = 0; d < D; ++d)
          x[d] = read_plain(p->q_dtype, src, ((size_t)i * (size_t)G + (size_t)g) * (size_t)D + (size_t)d);
        size_t plane = ((size_t)pb * 2 + (size_t)kv) * (size_t)G + (size_t)g;
        row_ctx c = {plane * (size_t)BS * (size_t)D, (size_t)D, t, BS, kv == 1};
        store_row(p->kv_dtype, scale, x, D, kv_data, kv_scales, row_elem, row_scale, &c);
      }
    }
    for (int d = 0; d < Di; ++d)
      x[d] = read_plain(p->index_q_dtype, ik_new, (size_t)i * (size_t)Di + (size_t)d);
    row_ctx c = {(size_t)pb * (size_t)BS * (size_t)Di, (size_t)Di, t, BS, 0};
    store_row(p->index_k_dtype, p->index_k_scale, x, Di, ik_data, ik_scales, row_elem, row_scale, &c);
  }
  free(x);
  return 0;
}
