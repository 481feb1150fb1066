// Host side of the C ABI declared in include/msa.h: argument validation
// (pure host code, before any HIP call), launch-geometry selection and
// dispatch to the kernels.  Between calls the library keeps per-thread state
// only (the error text, the opt-in profiling events) and per-device lookups
// (the compute-unit count, the no-allocation scratch address).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <string>

#include "launch.hpp"
#include "msa.h"

namespace {

thread_local std::string g_last_error;

msa_status_t fail(msa_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

msa_status_t ok() {
  g_last_error.clear();
  return MSA_SUCCESS;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int kMaxBlocksPerRow = 8192;  // top-k keeps a row's candidates in registers
constexpr int kMaxHpg = 16;             // heads of a group are MFMA columns (16 wide)
constexpr int kDecodeBlocksPerSplit = 4;

msa_status_t check_problem(const msa_problem_t *p, msa::Dims *d) {
  msa::profile_begin_call();
  if (p == nullptr) return fail(MSA_ERR_NULL_POINTER, "problem descriptor is NULL");
  if (p->num_seqs < 1) return fail(MSA_ERR_BAD_SHAPE, "num_seqs must be >= 1 (got %d)", p->num_seqs);
  if (p->num_q_heads < 1 || p->num_kv_groups < 1)
    return fail(MSA_ERR_BAD_SHAPE, "num_q_heads and num_kv_groups must be >= 1");
  if (p->num_q_heads % p->num_kv_groups != 0)
    return fail(MSA_ERR_BAD_SHAPE, "num_q_heads (%d) must be a multiple of num_kv_groups (%d)",
                p->num_q_heads, p->num_kv_groups);
  if (p->num_q_heads / p->num_kv_groups > kMaxHpg)
    return fail(MSA_ERR_BAD_SHAPE, "at most %d query heads per KV group are supported", kMaxHpg);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(MSA_ERR_BAD_SHAPE, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (p->idx_dim != 32 && p->idx_dim != 64 && p->idx_dim != 128)
    return fail(MSA_ERR_BAD_SHAPE, "idx_dim must be 32, 64 or 128 (got %d)", p->idx_dim);
  if (p->block_size != 64 && p->block_size != 128)
    return fail(MSA_ERR_BAD_SHAPE, "block_size must be 64 or 128 (got %d)", p->block_size);
  if (p->top_k < 1 || p->top_k > 64)
    return fail(MSA_ERR_BAD_SHAPE, "top_k must be in [1, 64] (got %d)", p->top_k);
  if (p->dtype != MSA_BF16 && p->dtype != MSA_F32)
    return fail(MSA_ERR_UNSUPPORTED_DTYPE, "dtype must be MSA_BF16 or MSA_F32 (got %d)", p->dtype);
  if (p->schedule < MSA_SCHED_AUTO || p->schedule > MSA_SCHED_KV_MAJOR)
    return fail(MSA_ERR_BAD_SHAPE, "unknown schedule %d", p->schedule);
  if (p->max_q_len < 0 || p->max_kv_len < 0 || p->total_q < 0 || p->total_kv < 0)
    return fail(MSA_ERR_BAD_SHAPE, "lengths must be non-negative");
  if (p->total_q < p->max_q_len || p->total_kv < p->max_kv_len)
    return fail(MSA_ERR_BAD_SHAPE, "total_q/total_kv must be >= max_q_len/max_kv_len");
  if (p->max_q_len > p->max_kv_len)
    return fail(MSA_ERR_BAD_SHAPE, "max_q_len (%d) exceeds max_kv_len (%lld)", p->max_q_len,
                (long long)p->max_kv_len);
  const int64_t nb = (p->max_kv_len + p->block_size - 1) / p->block_size;
  if (nb > kMaxBlocksPerRow)
    return fail(MSA_ERR_BAD_SHAPE, "ceil(max_kv_len / block_size) = %lld exceeds %d",
                (long long)nb, kMaxBlocksPerRow);
  if ((int64_t)p->num_seqs * p->num_kv_groups > 65535)
    return fail(MSA_ERR_BAD_SHAPE, "num_seqs * num_kv_groups must be <= 65535");
  if (p->total_q > (int64_t)INT32_MAX)
    return fail(MSA_ERR_BAD_SHAPE, "total_q must fit in int32 (got %lld)", (long long)p->total_q);
  if (!(p->softmax_scale > 0.f) || p->softmax_scale > 1e30f)
    return fail(MSA_ERR_BAD_SHAPE, "softmax_scale must be positive and finite");
  if (p->cu_q == nullptr || p->cu_kv == nullptr)
    return fail(MSA_ERR_NULL_POINTER, "cu_q and cu_kv must be device pointers");
  if (!aligned(p->cu_q, 8) || !aligned(p->cu_kv, 8))
    return fail(MSA_ERR_MISALIGNED, "cu_q and cu_kv must be 8-byte aligned");
  d->num_seqs = p->num_seqs;
  d->H = p->num_q_heads;
  d->G = p->num_kv_groups;
  d->d = p->head_dim;
  d->d_idx = p->idx_dim;
  d->B = p->block_size;
  d->top_k = p->top_k;
  d->max_q_len = p->max_q_len;
  d->max_kv_len = p->max_kv_len;
  d->total_q = p->total_q;
  d->total_kv = p->total_kv;
  d->nb_max = (int)nb;
  d->scale = p->softmax_scale;
  d->cu_q = p->cu_q;
  d->cu_kv = p->cu_kv;
  return MSA_SUCCESS;
}

msa_status_t check_tensor(const void *ptr, const char *name, bool needed) {
  if (!needed) return MSA_SUCCESS;
  if (ptr == nullptr) return fail(MSA_ERR_NULL_POINTER, "%s is NULL", name);
  if (!aligned(ptr, 16)) return fail(MSA_ERR_MISALIGNED, "%s must be 16-byte aligned", name);
  return MSA_SUCCESS;
}

msa_status_t launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MSA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

enum class AttnPath { kDecodeSplit, kQueryMajor, kKvMajor };

AttnPath attn_path(const msa_problem_t *p, const msa::Dims &d, int *n_split) {
  *n_split = 1;
  if (d.max_q_len == 1) {
    *n_split = (d.top_k + kDecodeBlocksPerSplit - 1) / kDecodeBlocksPerSplit;
    return AttnPath::kDecodeSplit;
  }
  if (p->dtype == MSA_BF16 && p->schedule != MSA_SCHED_QUERY_MAJOR &&
      d.total_kv <= (int64_t)INT32_MAX && msa::kvmajor_fits(d))
    return AttnPath::kKvMajor;
  return AttnPath::kQueryMajor;
}

size_t workspace_bytes(const msa_problem_t *p, const msa::Dims &d) {
  if (d.total_q == 0) return 0;  // nothing is launched
  int n_split = 1;
  switch (attn_path(p, d, &n_split)) {
    case AttnPath::kDecodeSplit:
      if (n_split <= 1) return 0;
      return (size_t)n_split * (size_t)d.total_q * (size_t)d.H * (size_t)(d.d + 1) * sizeof(float);
    case AttnPath::kKvMajor:  // one pass of the preferred size
      return msa::kvmajor_workspace_bytes(d, std::min(d.total_q, msa::kvmajor_preferred_rows(d)));
    case AttnPath::kQueryMajor:
      return 0;
  }
  return 0;
}

// The least workspace the call accepts: the KV-major path can run its rows in
// passes over one smaller workspace; every other path needs its full size.
size_t workspace_min_bytes(const msa_problem_t *p, const msa::Dims &d) {
  int n_split = 1;
  if (d.total_q > 0 && attn_path(p, d, &n_split) == AttnPath::kKvMajor)
    return msa::kvmajor_workspace_min_bytes(d);
  return workspace_bytes(p, d);
}

// With fixed_scratch, `workspace` is ignored: once every argument has been
// validated, the library's fixed device scratch (noalloc.hip) serves as the
// workspace, and a problem whose full-speed workspace (workspace_bytes)
// exceeds it is rejected.  Otherwise a workspace below that size (but at
// least the minimum) runs the KV-major path in passes of as many query rows
// as it holds; at or above it, in passes of the preferred size (one pass for
// all but long prefills).
msa_status_t attn_fwd(const msa_problem_t *prob, const void *q, const void *k, const void *v,
                      const int32_t *block_idx, void *out, float *lse, float *block_mass,
                      void *workspace, size_t workspace_bytes_given, void *stream,
                      bool fixed_scratch = false) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  const bool any_q = d.total_q > 0, any_kv = d.total_kv > 0;
  if ((st = check_tensor(q, "q", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(k, "k", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(v, "v", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(block_idx, "block_idx", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(out, "out", any_q)) != MSA_SUCCESS) return st;
  if (lse != nullptr && !aligned(lse, 4)) return fail(MSA_ERR_MISALIGNED, "lse must be 4-byte aligned");
  const size_t full = workspace_bytes(prob, d);
  size_t need = fixed_scratch ? full : workspace_min_bytes(prob, d);
  if (fixed_scratch) {
    const size_t have = msa::noalloc_scratch_bytes();
    if (need > have)
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                  "this problem needs %zu bytes of scratch; the fixed scratch of the "
                  "no-allocation call holds %zu (use msa_sparse_attn_fwd with a workspace)",
                  need, have);
    workspace = nullptr;
    workspace_bytes_given = have;
    if (need > 0 && d.total_q > 0) {
      const hipError_t e = msa::noalloc_scratch(&workspace);
      if (e != hipSuccess)
        return fail(MSA_ERR_DEVICE, "no-allocation scratch lookup: %s", hipGetErrorString(e));
    }
  }
  if (workspace_bytes_given < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes_given);
  if (need > 0 && workspace == nullptr) return fail(MSA_ERR_NULL_POINTER, "workspace is NULL");
  if (need > 0 && !aligned(workspace, 256))
    return fail(MSA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!any_q) return ok();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int n_split = 1;
  const AttnPath path = attn_path(prob, d, &n_split);
  if (path == AttnPath::kKvMajor) {
    const int64_t rows = std::min(msa::kvmajor_rows_per_pass(d, workspace_bytes_given),
                                  msa::kvmajor_preferred_rows(d));
    if (rows <= 0)  // cannot happen once the minimum is checked
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace holds no pass of query rows");
    return launched(msa::launch_attn_kvmajor_bf16(d, static_cast<const uint16_t *>(q),
                                                  static_cast<const uint16_t *>(k),
                                                  static_cast<const uint16_t *>(v), block_idx,
                                                  static_cast<uint16_t *>(out), lse, block_mass,
                                                  workspace, rows, s),
                    "attn_kvmajor");
  }
  float *part_o = nullptr, *part_lse = nullptr;
  if (n_split > 1) {
    part_o = static_cast<float *>(workspace);
    part_lse = part_o + (size_t)n_split * d.total_q * d.H * d.d;
  }
  hipError_t e;
  if (prob->dtype == MSA_F32)
    e = msa::launch_attn_qmajor_f32(d, static_cast<const float *>(q), static_cast<const float *>(k),
                                    static_cast<const float *>(v), block_idx,
                                    static_cast<float *>(out), lse, n_split, part_o, part_lse, s);
  else
    e = msa::launch_attn_qmajor_bf16(d, static_cast<const uint16_t *>(q),
                                     static_cast<const uint16_t *>(k),
                                     static_cast<const uint16_t *>(v), block_idx,
                                     static_cast<uint16_t *>(out), lse, n_split, part_o, part_lse, s);
  if (e != hipSuccess || n_split == 1) return launched(e, "attn_query_major");
  return launched(msa::launch_combine_splits(d, n_split, part_o, part_lse, out,
                                             prob->dtype == MSA_BF16, lse, s),
                  "attn_combine_splits");
}

}  // namespace

extern "C" {

msa_status_t msa_index_score(const msa_problem_t *prob, const void *q_idx, const void *k_idx,
                             float *scores, void *stream) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  const bool any_q = d.total_q > 0, any_kv = d.total_kv > 0;
  if ((st = check_tensor(q_idx, "q_idx", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(k_idx, "k_idx", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(scores, "scores", any_q && d.nb_max > 0)) != MSA_SUCCESS) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!any_q || d.nb_max == 0) return ok();
  if (prob->dtype == MSA_F32)
    return launched(msa::launch_index_score_f32(d, static_cast<const float *>(q_idx),
                                                static_cast<const float *>(k_idx), scores, s),
                    "index_score_f32");
  const uint16_t *qi = static_cast<const uint16_t *>(q_idx);
  const uint16_t *ki = static_cast<const uint16_t *>(k_idx);
  if (msa::decode_index_supported(d))
    return launched(msa::launch_index_score_decode_bf16(d, qi, ki, scores, s), "index_score_decode");
  return launched(msa::launch_index_score_bf16(d, qi, ki, scores, s), "index_score_mfma");
}

msa_status_t msa_topk_select(const msa_problem_t *prob, const float *scores, int32_t *block_idx,
                             void *stream) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  const bool any_q = d.total_q > 0;
  if ((st = check_tensor(scores, "scores", any_q && d.nb_max > 0)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(block_idx, "block_idx", any_q)) != MSA_SUCCESS) return st;
  if (!any_q) return ok();
  return launched(msa::launch_topk(d, scores, block_idx, reinterpret_cast<hipStream_t>(stream)),
                  "topk_select");
}

msa_status_t msa_index_topk_workspace_size(const msa_problem_t *prob, size_t *bytes) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (bytes == nullptr) return fail(MSA_ERR_NULL_POINTER, "bytes is NULL");
  *bytes = msa::index_topk_workspace_bytes(d);
  return ok();
}

msa_status_t msa_index_topk(const msa_problem_t *prob, const void *q_idx, const void *k_idx,
                            int32_t *block_idx, void *workspace, size_t workspace_bytes_given,
                            void *stream) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (prob->dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED_DTYPE, "the fused index scoring and Top-k takes bf16 inputs");
  const bool any_q = d.total_q > 0, any_kv = d.total_kv > 0;
  if ((st = check_tensor(q_idx, "q_idx", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(k_idx, "k_idx", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(block_idx, "block_idx", any_q)) != MSA_SUCCESS) return st;
  if (!msa::index_topk_supported(d))
    return fail(MSA_ERR_BAD_SHAPE, "the fused index scoring and Top-k holds at most 1024 "
                                   "candidates per row (segments x list length)");
  const size_t need = msa::index_topk_workspace_bytes(d);
  if (workspace_bytes_given < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes_given);
  if (need > 0 && workspace == nullptr) return fail(MSA_ERR_NULL_POINTER, "workspace is NULL");
  if (need > 0 && !aligned(workspace, 256))
    return fail(MSA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!any_q) return ok();
  return launched(msa::launch_index_topk(d, static_cast<const uint16_t *>(q_idx),
                                         static_cast<const uint16_t *>(k_idx), block_idx,
                                         workspace, reinterpret_cast<hipStream_t>(stream)),
                  "index_topk");
}

msa_status_t msa_index_topk_hier_workspace_size(const msa_problem_t *prob, int chunk_blocks,
                                               int keep_chunks, size_t *bytes) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (bytes == nullptr) return fail(MSA_ERR_NULL_POINTER, "bytes is NULL");
  if (!msa::hier_params_ok(d, chunk_blocks, keep_chunks))
    return fail(MSA_ERR_BAD_SHAPE,
                "chunk_blocks must be a power of two in [1, 64] and keep_chunks >= 1 with "
                "keep_chunks * chunk_blocks >= top_k - 1, (keep_chunks + 1) * chunk_blocks <= "
                "1024, ceil(NBmax / chunk_blocks) <= 1024 and num_seqs * that <= 16384");
  *bytes = msa::hier_workspace_bytes(d, chunk_blocks, keep_chunks);
  return ok();
}

msa_status_t msa_index_topk_hier(const msa_problem_t *prob, const void *q_idx, const void *k_idx,
                                 int chunk_blocks, int keep_chunks, int32_t *block_idx,
                                 int32_t *kept_chunks, void *workspace,
                                 size_t workspace_bytes_given, void *stream) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (prob->dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED_DTYPE, "the hierarchical selection takes bf16 inputs");
  size_t need = 0;
  if ((st = msa_index_topk_hier_workspace_size(prob, chunk_blocks, keep_chunks, &need)) !=
      MSA_SUCCESS)
    return st;
  const bool any_q = d.total_q > 0, any_kv = d.total_kv > 0;
  if ((st = check_tensor(q_idx, "q_idx", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(k_idx, "k_idx", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(block_idx, "block_idx", any_q)) != MSA_SUCCESS) return st;
  if (kept_chunks != nullptr && !aligned(kept_chunks, 4))
    return fail(MSA_ERR_MISALIGNED, "kept_chunks must be 4-byte aligned");
  if (workspace_bytes_given < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes_given);
  if (need > 0 && workspace == nullptr) return fail(MSA_ERR_NULL_POINTER, "workspace is NULL");
  if (need > 0 && !aligned(workspace, 256))
    return fail(MSA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!any_q) return ok();
  return launched(msa::launch_index_topk_hier(d, chunk_blocks, keep_chunks,
                                              static_cast<const uint16_t *>(q_idx),
                                              static_cast<const uint16_t *>(k_idx), block_idx,
                                              kept_chunks, workspace,
                                              reinterpret_cast<hipStream_t>(stream)),
                  "index_topk_hier");
}

msa_status_t msa_sparse_attn_workspace_size(const msa_problem_t *prob, size_t *bytes) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (bytes == nullptr) return fail(MSA_ERR_NULL_POINTER, "bytes is NULL");
  *bytes = workspace_bytes(prob, d);
  return ok();
}

msa_status_t msa_sparse_attn_workspace_size_min(const msa_problem_t *prob, size_t *bytes) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (bytes == nullptr) return fail(MSA_ERR_NULL_POINTER, "bytes is NULL");
  *bytes = workspace_min_bytes(prob, d);
  return ok();
}

msa_status_t msa_sparse_attn_rows_per_pass(const msa_problem_t *prob, size_t workspace_bytes_given,
                                           int64_t *rows) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (rows == nullptr) return fail(MSA_ERR_NULL_POINTER, "rows is NULL");
  *rows = 0;
  const size_t need = workspace_min_bytes(prob, d);
  if (workspace_bytes_given < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes_given);
  int n_split = 1;
  *rows = d.total_q > 0 && attn_path(prob, d, &n_split) == AttnPath::kKvMajor
              ? std::min(msa::kvmajor_rows_per_pass(d, workspace_bytes_given),
                         msa::kvmajor_preferred_rows(d))
              : d.total_q;
  return ok();
}

msa_status_t msa_sparse_attn_fwd(const msa_problem_t *prob, const void *q, const void *k,
                                 const void *v, const int32_t *block_idx, void *out, float *lse,
                                 void *workspace, size_t workspace_bytes_given, void *stream) {
  return attn_fwd(prob, q, k, v, block_idx, out, lse, nullptr, workspace, workspace_bytes_given,
                  stream);
}

msa_status_t msa_sparse_attn_fwd_noalloc(const msa_problem_t *prob, const void *q, const void *k,
                                         const void *v, const int32_t *block_idx, void *out,
                                         float *lse, void *stream) {
  return attn_fwd(prob, q, k, v, block_idx, out, lse, nullptr, nullptr, 0, stream, true);
}

msa_status_t msa_sparse_attn_fwd_mass(const msa_problem_t *prob, const void *q, const void *k,
                                      const void *v, const int32_t *block_idx, void *out,
                                      float *lse, float *block_mass, void *workspace,
                                      size_t workspace_bytes_given, void *stream) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (prob->dtype != MSA_BF16)
    return fail(MSA_ERR_UNSUPPORTED_DTYPE, "the block mass is computed by the bf16 KV-major path only");
  int n_split = 1;
  if (d.total_q > 0 && attn_path(prob, d, &n_split) != AttnPath::kKvMajor)
    return fail(MSA_ERR_BAD_SHAPE,
                "the block mass needs the KV-major schedule: multi-query rows (max_q_len > 1), "
                "schedule auto or kv_major, and a problem that schedule holds");
  if (d.total_q > 0 && block_mass == nullptr) return fail(MSA_ERR_NULL_POINTER, "block_mass is NULL");
  if (block_mass != nullptr && !aligned(block_mass, 4))
    return fail(MSA_ERR_MISALIGNED, "block_mass must be 4-byte aligned");
  return attn_fwd(prob, q, k, v, block_idx, out, lse, block_mass, workspace,
                  workspace_bytes_given, stream);
}

msa_status_t msa_indexer_kl(const msa_problem_t *prob, const float *scores, const int32_t *block_idx,
                            const float *block_mass, float *kl, float *grad, void *stream) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  const bool any = d.total_q > 0;
  if ((st = check_tensor(scores, "scores", any && d.nb_max > 0)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(block_idx, "block_idx", any)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(block_mass, "block_mass", any)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(kl, "kl", any)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(grad, "grad", any)) != MSA_SUCCESS) return st;
  if (!any) return ok();
  if (d.nb_max == 0) return fail(MSA_ERR_BAD_SHAPE, "no key blocks: max_kv_len is 0");
  return launched(msa::launch_indexer_kl(d, scores, block_idx, block_mass, kl, grad,
                                         reinterpret_cast<hipStream_t>(stream)),
                  "indexer_kl");
}

msa_status_t msa_indexer_bwd_workspace_size(const msa_problem_t *prob, size_t *bytes) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (bytes == nullptr) return fail(MSA_ERR_NULL_POINTER, "bytes is NULL");
  *bytes = msa::index_bwd_workspace_bytes(d);
  return ok();
}

msa_status_t msa_indexer_bwd(const msa_problem_t *prob, const void *q_idx, const void *k_idx,
                             const int32_t *block_idx, const float *grad, float *dq_idx,
                             float *dk_idx, void *workspace, size_t workspace_bytes_given,
                             void *stream) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  const bool any_q = d.total_q > 0, any_kv = d.total_kv > 0;
  if ((st = check_tensor(q_idx, "q_idx", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(k_idx, "k_idx", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(block_idx, "block_idx", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(grad, "grad", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(dq_idx, "dq_idx", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(dk_idx, "dk_idx", any_kv)) != MSA_SUCCESS) return st;
  if (d.total_q * (int64_t)d.top_k >= (int64_t)INT32_MAX)
    return fail(MSA_ERR_BAD_SHAPE, "total_q * top_k must be below 2^31");
  if (msa::index_bwd_hist_bytes(d) > 64 * 1024)
    return fail(MSA_ERR_BAD_SHAPE,
                "num_seqs * ceil(max_kv_len / block_size) must be at most 16384 for the "
                "index backward (one LDS histogram bin per (sequence, block))");
  const size_t need = msa::index_bwd_workspace_bytes(d);
  if (workspace_bytes_given < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes_given);
  if (need > 0 && workspace == nullptr) return fail(MSA_ERR_NULL_POINTER, "workspace is NULL");
  if (need > 0 && !aligned(workspace, 256))
    return fail(MSA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!any_q && !any_kv) return ok();
  // with no query row every key's gradient is 0: the launch only zero-fills dk_idx
  return launched(msa::launch_index_bwd(d, prob->dtype == MSA_BF16, q_idx, k_idx, block_idx, grad,
                                        dq_idx, dk_idx, workspace,
                                        reinterpret_cast<hipStream_t>(stream)),
                  "index_bwd");
}

namespace {
// The MFMA backward takes bf16 with head_dim 128, block_size 128 and 1, 2, 4,
// 8 or 16 heads per group; every other problem takes the plain FMA one.
bool attn_bwd_mfma(const msa_problem_t *prob, const msa::Dims &d) {
  return prob->dtype == MSA_BF16 && msa::attn_bwd_supported(d);
}
size_t attn_bwd_bytes(const msa_problem_t *prob, const msa::Dims &d) {
  return attn_bwd_mfma(prob, d) ? msa::attn_bwd_workspace_bytes(d, d.total_q)
                                : msa::attn_bwd_fma_workspace_bytes(d);
}
// The MFMA backward runs its rows in passes below its single-pass size; the
// FMA one needs its full workspace.
size_t attn_bwd_min_bytes(const msa_problem_t *prob, const msa::Dims &d) {
  return attn_bwd_mfma(prob, d) ? msa::attn_bwd_workspace_min_bytes(d)
                                : msa::attn_bwd_fma_workspace_bytes(d);
}
}  // namespace

msa_status_t msa_sparse_attn_bwd_workspace_size(const msa_problem_t *prob, size_t *bytes) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (bytes == nullptr) return fail(MSA_ERR_NULL_POINTER, "bytes is NULL");
  *bytes = attn_bwd_bytes(prob, d);
  return ok();
}

msa_status_t msa_sparse_attn_bwd_workspace_size_min(const msa_problem_t *prob, size_t *bytes) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (bytes == nullptr) return fail(MSA_ERR_NULL_POINTER, "bytes is NULL");
  *bytes = attn_bwd_min_bytes(prob, d);
  return ok();
}

msa_status_t msa_sparse_attn_bwd_rows_per_pass(const msa_problem_t *prob,
                                               size_t workspace_bytes_given, int64_t *rows) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  if (rows == nullptr) return fail(MSA_ERR_NULL_POINTER, "rows is NULL");
  *rows = 0;
  const size_t need = attn_bwd_min_bytes(prob, d);
  if (workspace_bytes_given < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes_given);
  *rows = attn_bwd_mfma(prob, d) && d.total_q > 0
              ? msa::attn_bwd_rows_per_pass(d, workspace_bytes_given)
              : d.total_q;
  return ok();
}

msa_status_t msa_sparse_attn_bwd(const msa_problem_t *prob, const void *q, const void *k,
                                 const void *v, const int32_t *block_idx, const void *out,
                                 const float *lse, const void *dout, float *dq, float *dk,
                                 float *dv, void *workspace, size_t workspace_bytes_given,
                                 void *stream) {
  msa::Dims d;
  msa_status_t st = check_problem(prob, &d);
  if (st != MSA_SUCCESS) return st;
  const bool any_q = d.total_q > 0, any_kv = d.total_kv > 0;
  if ((st = check_tensor(q, "q", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(k, "k", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(v, "v", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(block_idx, "block_idx", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(out, "out", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(lse, "lse", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(dout, "dout", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(dq, "dq", any_q)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(dk, "dk", any_kv)) != MSA_SUCCESS) return st;
  if ((st = check_tensor(dv, "dv", any_kv)) != MSA_SUCCESS) return st;
  if (d.total_q * (int64_t)d.top_k * d.H >= (int64_t)INT32_MAX)
    return fail(MSA_ERR_BAD_SHAPE, "total_q * top_k * num_q_heads must be below 2^31");
  if (msa::index_bwd_hist_bytes(d) > 64 * 1024)
    return fail(MSA_ERR_BAD_SHAPE,
                "num_seqs * ceil(max_kv_len / block_size) must be at most 16384 for the "
                "attention backward (one LDS histogram bin per (sequence, block))");
  const size_t need = attn_bwd_min_bytes(prob, d);
  if (workspace_bytes_given < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace_bytes_given);
  if (need > 0 && workspace == nullptr) return fail(MSA_ERR_NULL_POINTER, "workspace is NULL");
  if (need > 0 && !aligned(workspace, 256))
    return fail(MSA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (!any_q && !any_kv) return ok();
  if (!attn_bwd_mfma(prob, d))
    return launched(msa::launch_attn_bwd_fma(d, prob->dtype == MSA_BF16, q, k, v, block_idx, out,
                                             lse, dout, dq, dk, dv, workspace,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "attn_bwd_fma");
  return launched(msa::launch_attn_bwd_bf16(
                      d, static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                      static_cast<const uint16_t *>(v), block_idx,
                      static_cast<const uint16_t *>(out), lse,
                      static_cast<const uint16_t *>(dout), dq, dk, dv, workspace,
                      msa::attn_bwd_rows_per_pass(d, workspace_bytes_given),
                      reinterpret_cast<hipStream_t>(stream)),
                  "attn_bwd");
}

msa_status_t msa_debug_bounds_violations(uint64_t *violations, uint64_t *checks, int reset) {
  if (violations == nullptr) return fail(MSA_ERR_NULL_POINTER, "violations is NULL");
  *violations = 0;
  if (checks != nullptr) *checks = 0;
#ifdef MSA_DEBUG
  uint64_t c = 0, v = 0;
  const bool r = reset != 0;
  const bool read = msa::debug_counters_attn_kvmajor(&c, &v, r) &&
                    msa::debug_counters_attn_qmajor(&c, &v, r) &&
                    msa::debug_counters_attn_bwd(&c, &v, r) &&
                    msa::debug_counters_index_bwd(&c, &v, r) &&
                    msa::debug_counters_index_topk(&c, &v, r) &&
                    msa::debug_counters_index_hier(&c, &v, r);
  if (!read) return fail(MSA_ERR_DEVICE, "reading the debug counters failed");
  *violations = v;
  if (checks != nullptr) *checks = c;
  return ok();
#else
  (void)reset;
  return fail(MSA_ERR_NOT_AVAILABLE, "bounds counters exist only in the debug build (-DMSA_DEBUG)");
#endif
}

const char *msa_status_string(msa_status_t status) {
  switch (status) {
    case MSA_SUCCESS: return "success";
    case MSA_ERR_NULL_POINTER: return "null pointer";
    case MSA_ERR_BAD_SHAPE: return "unsupported or inconsistent shape";
    case MSA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case MSA_ERR_MISALIGNED: return "misaligned pointer";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MSA_ERR_DEVICE: return "device error";
    case MSA_ERR_NOT_AVAILABLE: return "not available in this library variant";
  }
  return "unknown status";
}

const char *msa_last_error_message(void) { return g_last_error.c_str(); }

int msa_abi_version(void) { return MSA_ABI_VERSION; }

}  // extern "C"
