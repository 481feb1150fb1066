/*
 * msa.h - C ABI of the MSA block-sparse attention library (gfx950 / MI355X).
 *
 * The library computes the three steps of MiniMax Sparse Attention as the
 * "MiniMax Sparse Attention" page (paper by Lai et al., 2026) describes them
 * in its Summary, second paragraph:
 *
 *   1. msa_index_score  - the Index Branch scores every key/value block by
 *                         max-pooling token-level dot products of an index
 *                         query with the block's index keys;
 *   2. msa_topk_select  - each GQA group keeps its own Top-k blocks; the
 *                         block holding the query's own position is always
 *                         kept (and counts as one of the k, as in the page's
 *                         Key points, "Benchmark configuration": B_k = 128
 *                         and k = 16 give 2,048 attended tokens);
 *   3. msa_sparse_attn_fwd - the Main Branch runs exact softmax attention
 *                         restricted to the kept blocks, for every query
 *                         head of the group (prefill and decode).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Sequences are packed back to back.  cu_q / cu_kv hold num_seqs + 1 row
 *    offsets (int64, DEVICE memory).  Sequence b owns query rows
 *    [cu_q[b], cu_q[b+1]) and key/value rows [cu_kv[b], cu_kv[b+1]).
 *  - Queries are the LAST len_q tokens of their sequence: local query i of
 *    sequence b sits at absolute position p = len_kv(b) - len_q(b) + i and
 *    sees keys 0..p (causal).  len_q(b) <= len_kv(b) is required; rows that
 *    break it are treated as having no causal key (scores -inf, no block
 *    kept, output 0, lse -inf) and never read out of bounds.
 *  - Blocks have block_size keys; block j of a sequence spans its keys
 *    [j*B, min((j+1)*B, len_kv)).  The current block of a query at p is
 *    J = floor(p / B).
 *  - Query head h belongs to KV group h / (H / G) (contiguous GQA groups).
 *  - Layouts (row-major, innermost last, no padding between rows):
 *        q, out  [total_q,  H, d]        k, v   [total_kv, G, d]
 *        q_idx   [total_q,  G, d_idx]    k_idx  [total_kv, G, d_idx]
 *        scores  [G, total_q, NBmax] fp32, NBmax = ceil(max_kv_len / B)
 *        block_idx [G, total_q, top_k] int32
 *        lse     [total_q, H] fp32
 *    Element type of q, k, v, q_idx, k_idx and out is `dtype` (bf16 or
 *    fp32).  Every device pointer must be 16-byte aligned.
 *  - Every pointer is DEVICE memory unless marked "host".  The caller owns
 *    and frees all memory; the library never allocates, frees, copies to the
 *    host or synchronises.  Calls are asynchronous on `stream` (a
 *    hipStream_t; NULL = the default stream).
 *  - Errors: all arguments are validated on the host before anything is
 *    launched; on any error nothing is launched, outputs are untouched and
 *    a status != MSA_SUCCESS is returned (details in
 *    msa_last_error_message(), per thread).  A failed launch returns
 *    MSA_ERR_DEVICE.  Faults inside kernels surface at the caller's next
 *    synchronisation.  Inputs holding NaN or Inf give unspecified values
 *    (but no out-of-bounds access).
 *  - Supported shapes: head_dim d in {64, 128}; idx_dim d_idx in {32, 64,
 *    128}; block_size in {64, 128}; H % G == 0 with 1 <= H/G <= 16;
 *    1 <= top_k <= 64; NBmax <= 8192.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 1

typedef enum {
  MSA_SUCCESS = 0,
  MSA_ERR_NULL_POINTER = 1,
  MSA_ERR_BAD_SHAPE = 2,
  MSA_ERR_UNSUPPORTED_DTYPE = 3,
  MSA_ERR_MISALIGNED = 4,
  MSA_ERR_WORKSPACE_TOO_SMALL = 5,
  MSA_ERR_DEVICE = 6,
  MSA_ERR_NOT_AVAILABLE = 7 /* the entry point is not part of this library variant */
} msa_status_t;

typedef enum { MSA_BF16 = 0, MSA_F32 = 1 } msa_dtype_t;

/* How msa_sparse_attn_fwd orders its work for multi-query (prefill) rows.
 * Both give the same result up to fp32 rounding order. */
typedef enum {
  MSA_SCHED_AUTO = 0,        /* library choice (KV-major for bf16 prefill) */
  MSA_SCHED_QUERY_MAJOR = 1, /* one work item per (query, group): gathers its k blocks */
  MSA_SCHED_KV_MAJOR = 2     /* one work item per (group, kept block, query chunk),
                                then a per-query merge (bf16 only; used while
                                total_q < 2^25, total_kv < 2^31,
                                top_k * H <= 8000 and the (query, group, kept
                                block) entries number fewer than about 2^31;
                                query-major beyond) */
} msa_schedule_t;

typedef struct {
  int32_t num_seqs;        /* >= 1 */
  int32_t num_q_heads;     /* H */
  int32_t num_kv_groups;   /* G */
  int32_t head_dim;        /* d */
  int32_t idx_dim;         /* d_idx */
  int32_t block_size;      /* B */
  int32_t top_k;           /* k, counts the always-kept current block */
  int32_t dtype;           /* msa_dtype_t */
  int32_t schedule;        /* msa_schedule_t (attention only) */
  int32_t max_q_len;       /* host: max over sequences of len_q */
  int64_t max_kv_len;      /* host: max over sequences of len_kv */
  int64_t total_q;         /* host: cu_q[num_seqs] */
  int64_t total_kv;        /* host: cu_kv[num_seqs] */
  float softmax_scale;     /* multiplies q.k before the softmax (e.g. 1/sqrt(d)) */
  const int64_t *cu_q;     /* device [num_seqs + 1] */
  const int64_t *cu_kv;    /* device [num_seqs + 1] */
} msa_problem_t;

/* Step 1 - Index Branch block scores.
 * scores[g, r, j] = max over keys s of block j with s <= p(r) of
 *                   sum_c q_idx[r, g, c] * k_idx[s, g, c]   (fp32 accumulate)
 * and -inf for every j > J(r) up to NBmax - 1.  No scale is applied.
 * bf16 inputs use bf16 MFMA products (exact in fp32) with fp32 sums. */
msa_status_t msa_index_score(const msa_problem_t *prob, const void *q_idx, const void *k_idx,
                             float *scores, void *stream);

/* Step 2 - per-group Top-k with the current block forced.
 * For row r with current block J: if J <= k-1 the kept set is {0..J};
 * otherwise the k-1 best of blocks 0..J-1 by (score descending, block index
 * ascending) plus J.  block_idx[g, r, :] lists the kept blocks ascending
 * (so J is the last valid entry) and pads with -1.  Exact on the fp32
 * scores it is given: pure comparisons, no exponentials. */
msa_status_t msa_topk_select(const msa_problem_t *prob, const float *scores, int32_t *block_idx,
                             void *stream);

/* Steps 1 and 2 fused, without the score tensor: block_idx as msa_topk_select
 * would produce it from msa_index_score's scores, bit for bit (the same MFMA
 * arithmetic scores every candidate block, and the same selection rule keeps
 * them).  The scores themselves are never written to memory: per tile of 512
 * queries and segment of key blocks, each query keeps its best candidates
 * (score descending, then block index ascending; at least top_k - 1 of them)
 * as the blocks stream by, and a merge over the segments lists the final
 * blocks ascending with the current block appended.  This follows the page's
 * selection (Summary, paragraph 2) and its comparison-only Top-k (Summary,
 * paragraph 3), and removes the O(L^2) score round trip that the LongCat
 * Sparse Attention page names as the indexer's cost (Abstract).  Let L be
 * top_k - 1 rounded up to a power of two (at least 4): segments are 8 L
 * blocks long, and ceil(NBmax / (8 L)) * L <= 1024 is required (every
 * NBmax <= 8192 fits; else MSA_ERR_BAD_SHAPE).  bf16 only (else
 * MSA_ERR_UNSUPPORTED_DTYPE).  `workspace` must hold
 * msa_index_topk_workspace_size() bytes (G * total_q * segments * L 8-byte
 * keys, a quarter of the score tensor), 256-byte aligned; its contents need
 * no initialisation. */
msa_status_t msa_index_topk_workspace_size(const msa_problem_t *prob, size_t *bytes);
msa_status_t msa_index_topk(const msa_problem_t *prob, const void *q_idx, const void *k_idx,
                            int32_t *block_idx, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Hierarchical (coarse-to-fine) selection: an APPROXIMATION of steps 1 and 2
 * that scores only a narrowed candidate set (the "LongCat Sparse Attention"
 * page, Abstract, strategy (3): a coarse-to-fine scoring scheme narrows each
 * query's candidates to cut the indexing computation; the page gives no
 * formula, and this is the reading taken).  Chunks of chunk_blocks (S)
 * consecutive blocks carry a coarse key, the mean of their B * S index keys
 * (full chunks only).  For a query at position p with current block J and
 * current chunk cJ = J / S:
 *   - every chunk c < cJ scores <q_idx, coarse key of c> (fp32);
 *   - the keep_chunks (C) best are kept (score descending, chunk ascending;
 *     all of them when cJ <= C);
 *   - the blocks of the kept chunks and the blocks cJ * S .. J-1 get the
 *     exact max-pooled block score of msa_index_score;
 *   - the k-1 best of those (score descending, block ascending) and J are
 *     kept; rows with J <= k-1 keep 0..J.
 * With C >= the number of chunks this equals msa_topk_select on
 * msa_index_score's scores.  block_idx [G, total_q, top_k] as msa_topk_select
 * (ascending, -1 padded); kept_chunks (optional, may be NULL) [G, total_q, C]
 * int32 the kept chunks ascending, -1 padded (rows at negative positions get
 * -1).  Requirements: bf16 (else MSA_ERR_UNSUPPORTED_DTYPE); S a power of two
 * in [1, 64]; C >= 1 with C * S >= top_k - 1; (C + 1) * S <= 1024;
 * ceil(NBmax / S) <= 1024 and num_seqs * ceil(NBmax / S) <= 16384 (else
 * MSA_ERR_BAD_SHAPE).  `workspace` must hold
 * msa_index_topk_hier_workspace_size() bytes, 256-byte aligned; its contents
 * need no initialisation. */
msa_status_t msa_index_topk_hier_workspace_size(const msa_problem_t *prob, int chunk_blocks,
                                               int keep_chunks, size_t *bytes);
msa_status_t msa_index_topk_hier(const msa_problem_t *prob, const void *q_idx, const void *k_idx,
                                 int chunk_blocks, int keep_chunks, int32_t *block_idx,
                                 int32_t *kept_chunks, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Bytes of device workspace with which msa_sparse_attn_fwd runs this
 * problem and schedule at full speed (0 is possible); a larger workspace is
 * not used.  Writes the size to *bytes (host).  On the KV-major schedule
 * (multi-query bf16 rows) long prefills run in consecutive passes over the
 * query rows: at most as many rows per pass as make the gathered query rows
 * of one group about 32 MiB (16,384 rows at H/G = 8 and d = 128), so that a
 * pass's rows stay cached between their many reads; this size holds one such
 * pass (all rows of shorter problems: one pass).  The outputs are identical
 * bit for bit whatever the passes. */
msa_status_t msa_sparse_attn_workspace_size(const msa_problem_t *prob, size_t *bytes);

/* The least workspace msa_sparse_attn_fwd and msa_sparse_attn_fwd_mass
 * accept for this problem and schedule (host *bytes).  It equals
 * msa_sparse_attn_workspace_size() except on the KV-major schedule, whose
 * workspace grows with the rows of a pass times top_k * num_q_heads *
 * head_dim (the per-slot partial results): given less than
 * msa_sparse_attn_workspace_size(), that schedule runs the query rows in
 * consecutive passes of as many rows as the workspace holds (at least 256
 * rows, or all of them), reusing it for every pass.  Each pass re-reads the
 * K/V blocks its rows keep; the outputs are identical bit for bit. */
msa_status_t msa_sparse_attn_workspace_size_min(const msa_problem_t *prob, size_t *bytes);

/* Query rows per pass that msa_sparse_attn_fwd (or _mass) runs with a
 * workspace of `workspace_bytes` (host *rows): the rows it holds, at most the
 * preferred pass size of msa_sparse_attn_workspace_size(); total_q when the
 * schedule is not KV-major.  MSA_ERR_WORKSPACE_TOO_SMALL (and *rows = 0)
 * below msa_sparse_attn_workspace_size_min(). */
msa_status_t msa_sparse_attn_rows_per_pass(const msa_problem_t *prob, size_t workspace_bytes,
                                           int64_t *rows);

/* Step 3 - exact softmax attention over the kept blocks.
 * For query row r, head h of group g: keys = every s <= p(r) inside a block
 * listed in block_idx[g, r, :] (entries < 0 are ignored; entries must be
 * distinct and <= J(r)); z_s = softmax_scale * q[r,h].k[s,g];
 * out[r,h] = sum_s exp(z_s - m) v[s,g] / sum_s exp(z_s - m), m = max z.
 * If lse is not NULL, lse[r,h] = m + ln(sum_s exp(z_s - m)).
 * Rows with max_q_len == 1 use the split-KV decode kernels.  out has the
 * input dtype (bf16 rounding to nearest even).  `workspace` must hold at
 * least msa_sparse_attn_workspace_size_min() bytes (it may be NULL if that
 * is 0; workspace_bytes is its size, and a workspace below
 * msa_sparse_attn_workspace_size() runs the KV-major schedule in smaller
 * passes);
 * its contents need no initialisation and are clobbered. */
msa_status_t msa_sparse_attn_fwd(const msa_problem_t *prob, const void *q, const void *k,
                                 const void *v, const int32_t *block_idx, void *out, float *lse,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* msa_sparse_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, same kernels and same results as
 * msa_sparse_attn_fwd, without a workspace: the call uses a fixed scratch
 * array of 64 MiB that the library holds on every GPU it runs on until the
 * process ends.  It allocates and frees nothing, and runs as
 * msa_sparse_attn_fwd does with msa_sparse_attn_workspace_size() bytes.  A
 * problem whose msa_sparse_attn_workspace_size() exceeds 64 MiB is rejected
 * with MSA_ERR_WORKSPACE_TOO_SMALL before anything is launched (use
 * msa_sparse_attn_fwd for those).  All calls on one GPU share the scratch:
 * calls that overlap in time on one GPU (on different streams) race and
 * must be serialised by the caller; consecutive calls need no clearing. */
msa_status_t msa_sparse_attn_fwd_noalloc(const msa_problem_t *prob, const void *q, const void *k,
                                         const void *v, const int32_t *block_idx, void *out,
                                         float *lse, void *stream);

/* Training support: the target and loss of the indexer's KL objective.  The
 * page (Summary, paragraph 2) trains the Index Branch through a KL
 * objective matched to the group-averaged Main Branch distribution, with
 * the Main Branch detached, because Top-k selection has no gradient.  The
 * two calls below take that objective as: p = the Main Branch's attention
 * mass on each kept block, averaged over the group's heads; q = the softmax
 * of the raw block scores over the same kept blocks; loss KL(p || q) per
 * (group, row); the gradient flows into the scores only. */

/* msa_sparse_attn_fwd plus the Main Branch block mass:
 *   block_mass[g, r, i] = (1/(H/G)) * sum over heads h of group g of the
 *                         attention weight head h puts on the causal keys of
 *                         block block_idx[g, r, i]
 * (0 for padding slots and for rows without causal keys; each other row
 * sums to 1).  It comes out of the KV-major combine of the per-block (max,
 * sum) pairs, so it costs one extra fp32 store per kept slot.  Requirements
 * beyond msa_sparse_attn_fwd: dtype MSA_BF16 (else
 * MSA_ERR_UNSUPPORTED_DTYPE); the KV-major schedule, i.e. max_q_len > 1,
 * schedule AUTO or KV_MAJOR and a problem that schedule holds (else
 * MSA_ERR_BAD_SHAPE); block_mass [G, total_q, top_k] fp32, 4-byte aligned,
 * not NULL when total_q > 0.  Same workspace as msa_sparse_attn_fwd. */
msa_status_t msa_sparse_attn_fwd_mass(const msa_problem_t *prob, const void *q, const void *k,
                                      const void *v, const int32_t *block_idx, void *out,
                                      float *lse, float *block_mass, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* KL objective of the Index Branch over the kept blocks, and its gradient
 * in the block scores with the target held fixed.  For row r of group g,
 * kept slots i are those with 0 <= block_idx[g, r, i] < NBmax, and
 * p_i = block_mass[g, r, i]:
 *   q_i            = exp(s_i) / sum_i' exp(s_i'),  s_i = scores[g, r, block_idx[g, r, i]]
 *   kl[g, r]       = sum_i p_i (ln p_i - ln q_i)       (terms with p_i = 0 are 0)
 *   grad[g, r, i]  = q_i * sum_i' p_i' - p_i           (= d kl[g, r] / d s_i)
 * Padding slots get grad 0; a row without kept blocks gets kl 0.  fp32
 * throughout (scores from msa_index_score, block_mass from
 * msa_sparse_attn_fwd_mass, either dtype).  Shapes: scores [G, total_q,
 * NBmax], block_idx and block_mass and grad [G, total_q, top_k], kl
 * [G, total_q]. */
msa_status_t msa_indexer_kl(const msa_problem_t *prob, const float *scores,
                            const int32_t *block_idx, const float *block_mass, float *kl,
                            float *grad, void *stream);

/* Backward of the Index Branch max-pooling (page: Summary, paragraph 2; the
 * block score is the maximum of token-level dot products, so a kept block's
 * score gradient reaches only the causal key that attains that maximum).
 * grad[g, r, i] is the gradient of the score of kept slot i of row r
 * (msa_indexer_kl's grad, or any other); with a = the arg-max key of block
 * block_idx[g, r, i] over the keys s <= p(r) of that block:
 *   dq_idx[r, g] = sum over slots i (in slot order) of grad[g,r,i] * k_idx[a, g]
 *   dk_idx[s, g] = sum over (r, i) with a = s (in (r, i) order) of grad[g,r,i] * q_idx[r, g]
 * Slots that are padding or whose block holds no causal key add nothing;
 * keys that no slot takes get 0.  The arg-max is an integer decided by
 * floating point: each dot product is summed in fp32 in channel order
 * (every product rounded to fp32, then added), ties to the lower key; where
 * two keys' exact dot products lie within that fp32 rounding of each other,
 * either may be taken.
 * Sums are fp32, deterministic (no floating-point atomics).  q_idx, k_idx
 * have the problem's dtype; grad [G, total_q, top_k], dq_idx [total_q, G,
 * d_idx] and dk_idx [total_kv, G, d_idx] are fp32, fully written.
 * Requirements beyond the common ones: total_q * top_k < 2^31 and
 * num_seqs * NBmax <= 16384 (else MSA_ERR_BAD_SHAPE).  `workspace` must
 * hold msa_indexer_bwd_workspace_size() bytes, 256-byte aligned. */
msa_status_t msa_indexer_bwd_workspace_size(const msa_problem_t *prob, size_t *bytes);
msa_status_t msa_indexer_bwd(const msa_problem_t *prob, const void *q_idx, const void *k_idx,
                             const int32_t *block_idx, const float *grad, float *dq_idx,
                             float *dk_idx, void *workspace, size_t workspace_bytes,
                             void *stream);

/* Backward of the Main Branch attention (page: Summary, paragraph 2; exact
 * softmax attention over the keys of the kept blocks, so its gradient is
 * that of dense attention restricted to the same keys).  Inputs are those of
 * msa_sparse_attn_fwd plus its results and the upstream gradient: out
 * [total_q, H, d] and lse [total_q, H] from msa_sparse_attn_fwd (or
 * msa_sparse_attn_fwd_mass) on the same q, k, v and block_idx, and dout
 * [total_q, H, d].  With P the attention weights (rebuilt as
 * exp(z - lse)), D = <dout, out> and dS_s = P_s (<dout, v_s> - D):
 *   dq[t, h]  = scale * sum_s dS_s k[s, g]
 *   dk[s, g]  = scale * sum over (t, h of g) keeping s of dS_s q[t, h]
 *   dv[s, g]  = sum over (t, h of g) keeping s of P_s dout[t, h]
 * Rows without a kept causal key get dq 0; keys that no row keeps get dk and
 * dv 0.  q, k, v, out and dout have the problem's dtype; dq [total_q, H, d],
 * dk and dv [total_kv, G, d] are fp32, fully written.  Sums are fp32 and
 * deterministic (no floating-point atomics).  bf16 problems with head_dim
 * 128, block_size 128 and H/G in {1, 2, 4, 8, 16} run on the matrix cores,
 * rounding P and dS to bf16 for the products that use them and each slot's
 * share of dq to bf16 before the slots are added; every other problem runs
 * plain fp32 multiply-adds.  Requirements beyond the common ones:
 * total_q * top_k * H < 2^31 and num_seqs * NBmax <= 16384 (else
 * MSA_ERR_BAD_SHAPE).  All tensors 16-byte aligned; `workspace` must hold
 * at least msa_sparse_attn_bwd_workspace_size_min() bytes, 256-byte
 * aligned.  msa_sparse_attn_bwd_workspace_size() is the single-pass size;
 * the matrix-core backward's workspace grows with total_q * top_k *
 * num_q_heads * head_dim (each kept slot's share of dq), and given less it
 * runs the query rows in consecutive passes of as many rows as fit (at
 * least 256, or all of them).  dq is then identical bit for bit; dk and dv
 * add the passes' sums in pass order (deterministic, rounded differently
 * from a single pass). */
msa_status_t msa_sparse_attn_bwd_workspace_size(const msa_problem_t *prob, size_t *bytes);
msa_status_t msa_sparse_attn_bwd_workspace_size_min(const msa_problem_t *prob, size_t *bytes);
/* Query rows per pass of msa_sparse_attn_bwd with a workspace of
 * `workspace_bytes` (host *rows; total_q for one pass or the FMA backward);
 * MSA_ERR_WORKSPACE_TOO_SMALL (and *rows = 0) below the minimum. */
msa_status_t msa_sparse_attn_bwd_rows_per_pass(const msa_problem_t *prob, size_t workspace_bytes,
                                               int64_t *rows);
msa_status_t msa_sparse_attn_bwd(const msa_problem_t *prob, const void *q, const void *k,
                                 const void *v, const int32_t *block_idx, const void *out,
                                 const float *lse, const void *dout, float *dq, float *dk,
                                 float *dv, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Kernel timing hook (diagnostics).  After this call, every msa_* call on
 * the calling thread records events[i] (each a hipEvent_t created by the
 * caller) on its stream right after launching its i-th kernel, for i <
 * num_events; the count restarts at each call.  Pass NULL / 0 to turn it
 * off.  The caller keeps ownership of the events and of the array, which
 * must stay valid while the hook is set. */
void msa_set_profile_events(void *const *events, int num_events);

/* Gather bounds counters (diagnostics; debug builds only).  The debug build
 * of the library (libmsa_debug.so, compiled with -DMSA_DEBUG) checks every
 * index that a kernel reads from memory and then follows: the block lists
 * of the query-major attention, the bucket entries and work-item
 * descriptors of the KV-major attention and of both backward passes, the
 * candidate lists of the fused selection and the chunk lists of the
 * hierarchical one.  Each index is checked against the buffer it addresses
 * and against what the method fixes for it (the entry's query belongs to
 * the bucket's sequence, the block is causal for it, a list holds no more
 * than its capacity).  Every check adds one per lane to a device count of
 * checks, and a failed one also to a count of violations; the access
 * itself is not changed, so the debug build reports bookkeeping errors
 * that read valid memory with the wrong meaning, and cannot prevent a
 * fault from one that leaves the allocation.  This call writes the
 * violations on the current device to *violations (host) and, when
 * `checks` (host) is not NULL, the checks to *checks; nonzero `reset`
 * clears both counts.  It copies from the device: synchronise the streams
 * of earlier calls first.  The release library returns
 * MSA_ERR_NOT_AVAILABLE and writes 0. */
msa_status_t msa_debug_bounds_violations(uint64_t *violations, uint64_t *checks, int reset);

/* Static text for a status code. */
const char *msa_status_string(msa_status_t status);
/* Detail of the last failure on the calling thread ("" if none). */
const char *msa_last_error_message(void);
/* MSA_ABI_VERSION of the loaded library. */
int msa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */
