// Internal host-side launch entry points of the kernels (not part of the C ABI).
// Every function launches asynchronously on `stream` and returns the status of
// the launch itself (hipGetLastError after the launch).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Timing hook (profile.cpp): reset at the start of each public call, marked
// after every kernel launch.
void profile_begin_call();
void profile_mark(hipStream_t s);

// Debug builds: per-source-file device counters of the gather bounds checks
// (MSA_DCHECK) on the current device: lanes that checked and lanes that
// failed are added to *checks and *violations; `reset` clears them after
// reading.  false if the device could not be read.
#ifdef MSA_DEBUG
bool debug_counters_attn_kvmajor(uint64_t *checks, uint64_t *violations, bool reset);
bool debug_counters_attn_qmajor(uint64_t *checks, uint64_t *violations, bool reset);
bool debug_counters_attn_bwd(uint64_t *checks, uint64_t *violations, bool reset);
bool debug_counters_index_bwd(uint64_t *checks, uint64_t *violations, bool reset);
bool debug_counters_index_topk(uint64_t *checks, uint64_t *violations, bool reset);
bool debug_counters_index_hier(uint64_t *checks, uint64_t *violations, bool reset);
#endif

struct Dims {
  int num_seqs, H, G, d, d_idx, B, top_k;
  int max_q_len;
  int64_t max_kv_len, total_q, total_kv;
  int nb_max;          // ceil(max_kv_len / B): score row stride
  float scale;
  const int64_t *cu_q, *cu_kv;
};

// Index Branch block scores.
hipError_t launch_index_score_bf16(const Dims &p, const uint16_t *q_idx, const uint16_t *k_idx,
                                   float *scores, hipStream_t s);
hipError_t launch_index_score_decode_bf16(const Dims &p, const uint16_t *q_idx,
                                          const uint16_t *k_idx, float *scores, hipStream_t s);
bool decode_index_supported(const Dims &p);
hipError_t launch_index_score_f32(const Dims &p, const float *q_idx, const float *k_idx,
                                  float *scores, hipStream_t s);

// Index scoring fused with the Top-k (index_topk.hip): per (query tile, key
// segment) the k-1 best candidates, then a per-row merge.
int index_topk_segment(const Dims &p);
int index_topk_nseg(const Dims &p);
size_t index_topk_workspace_bytes(const Dims &p);
bool index_topk_supported(const Dims &p);
hipError_t launch_index_topk(const Dims &p, const uint16_t *q_idx, const uint16_t *k_idx,
                             int32_t *block_idx, void *workspace, hipStream_t s);

// Hierarchical (coarse-to-fine) selection (index_hier.hip).
bool hier_params_ok(const Dims &p, int chunk_blocks, int keep_chunks);
size_t hier_workspace_bytes(const Dims &p, int chunk_blocks, int keep_chunks);
hipError_t launch_index_topk_hier(const Dims &p, int chunk_blocks, int keep_chunks,
                                  const uint16_t *q_idx, const uint16_t *k_idx,
                                  int32_t *block_idx, int32_t *kept_chunks, void *workspace,
                                  hipStream_t s);

// Top-k with the current block forced.
hipError_t launch_topk(const Dims &p, const float *scores, int32_t *block_idx, hipStream_t s);

// Attention, query-major (one work item per query row, group and split).
// With n_split > 1 the splits write normalised partials to `part_o`
// [n_split, total_q, H, d] fp32 and `part_lse` [n_split, total_q, H] and
// launch_combine_splits merges them.
hipError_t launch_attn_qmajor_bf16(const Dims &p, const uint16_t *q, const uint16_t *k,
                                   const uint16_t *v, const int32_t *block_idx, uint16_t *out,
                                   float *lse, int n_split, float *part_o, float *part_lse,
                                   hipStream_t s);
hipError_t launch_attn_qmajor_f32(const Dims &p, const float *q, const float *k, const float *v,
                                  const int32_t *block_idx, float *out, float *lse, int n_split,
                                  float *part_o, float *part_lse, hipStream_t s);
hipError_t launch_combine_splits(const Dims &p, int n_split, const float *part_o,
                                 const float *part_lse, void *out, bool out_bf16, float *lse,
                                 hipStream_t s);

// Attention, KV-major prefill (bf16): see attn_kvmajor.hip.  The query rows
// run in passes of rows_per_pass rows that share one workspace of
// kvmajor_workspace_bytes(p, rows_per_pass) bytes; kvmajor_rows_per_pass
// gives the most rows a workspace holds (0 if not even the fewest,
// kvmajor_workspace_min_bytes).  kvmajor_fits: the schedule's 32-bit entry
// and item indices hold this problem.  block_mass (may be NULL):
// [G, total_q, top_k] Main Branch mass per kept slot.
bool kvmajor_fits(const Dims &p);
size_t kvmajor_workspace_bytes(const Dims &p, int64_t rows_per_pass);
size_t kvmajor_workspace_min_bytes(const Dims &p);
int64_t kvmajor_rows_per_pass(const Dims &p, size_t workspace_bytes);
// The most rows per pass the path uses (a pass of them stays cached); a
// larger workspace changes nothing.
int64_t kvmajor_preferred_rows(const Dims &p);
hipError_t launch_attn_kvmajor_bf16(const Dims &p, const uint16_t *q, const uint16_t *k,
                                    const uint16_t *v, const int32_t *block_idx, uint16_t *out,
                                    float *lse, float *block_mass, void *workspace,
                                    int64_t rows_per_pass, hipStream_t s);

// Backward of the Index Branch max-pooling (index_bwd.hip).
size_t index_bwd_workspace_bytes(const Dims &p);
int64_t index_bwd_hist_bytes(const Dims &p);  // LDS of its per-tile bucket histogram
hipError_t launch_index_bwd(const Dims &p, bool bf16, const void *q_idx, const void *k_idx,
                            const int32_t *block_idx, const float *grad, float *dq_idx,
                            float *dk_idx, void *workspace, hipStream_t s);

// Backward of the Main Branch attention, bf16 (attn_bwd.hip).
bool attn_bwd_supported(const Dims &p);  // head dim 128, block size 128, 64 % (H/G) == 0
// The query rows run in passes of rows_per_pass rows over one workspace of
// attn_bwd_workspace_bytes(p, rows_per_pass) bytes (the per-slot dQ shares
// and item partials of one pass); attn_bwd_rows_per_pass gives the most rows
// a workspace holds (0 below attn_bwd_workspace_min_bytes).
size_t attn_bwd_workspace_bytes(const Dims &p, int64_t rows_per_pass);
size_t attn_bwd_workspace_min_bytes(const Dims &p);
int64_t attn_bwd_rows_per_pass(const Dims &p, size_t workspace_bytes);
hipError_t launch_attn_bwd_bf16(const Dims &p, const uint16_t *q, const uint16_t *k,
                                const uint16_t *v, const int32_t *block_idx, const uint16_t *out,
                                const float *lse, const uint16_t *dout, float *dq, float *dk,
                                float *dv, void *workspace, int64_t rows_per_pass,
                                hipStream_t s);

// The same backward with plain fp32 FMA for every other shape and dtype
// (attn_bwd_fma.hip).
size_t attn_bwd_fma_workspace_bytes(const Dims &p);
hipError_t launch_attn_bwd_fma(const Dims &p, bool bf16, const void *q, const void *k,
                               const void *v, const int32_t *block_idx, const void *out,
                               const float *lse, const void *dout, float *dq, float *dk,
                               float *dv, void *workspace, hipStream_t s);

// Fixed device scratch of the no-allocation attention entry point
// (noalloc.hip): its size, and its device address on the current device
// (looked up once per device with hipGetSymbolAddress).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void **ptr);

// Indexer KL objective over the kept blocks (indexer_kl.hip).
hipError_t launch_indexer_kl(const Dims &p, const float *scores, const int32_t *block_idx,
                             const float *block_mass, float *kl, float *grad, hipStream_t s);

}  // namespace msa
