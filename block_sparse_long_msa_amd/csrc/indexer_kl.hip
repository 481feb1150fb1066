// Indexer KL objective over the kept blocks ("MiniMax Sparse Attention" page,
// Summary, paragraph 2: since Top-k selection has no gradient, the Index
// Branch learns through a KL objective matched to the group-averaged Main
// Branch distribution, with the Main Branch detached).  Per (group g, row r)
// with kept slots i (0 <= block_idx[g, r, i] < NBmax):
//   q_i         = softmax over the kept slots of scores[g, r, block_idx[g, r, i]]
//   kl[g, r]    = sum_i p_i (ln p_i - ln q_i)   with p = block_mass, 0 ln 0 = 0
//   grad[g,r,i] = q_i * sum_i' p_i' - p_i      (d kl / d score, p held fixed)
// Padding slots get grad 0; a row without kept blocks (or whose kept scores
// are all -inf) gets kl 0 and zero gradients.
//
// Rows are packed SEG = 16, 32 or 64 lanes apart (the smallest that holds k
// slots), so one wave handles 64 / SEG rows of one group, one lane per slot;
// reductions stay inside a row's lane segment.  The work is k gathered
// scores and k masses per row: a small, latency-bound kernel next to the
// forward pass.
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

template <int SEG>
__device__ __forceinline__ float seg_max(float v) {
#pragma unroll
  for (int off = SEG / 2; off >= 1; off >>= 1) v = fmaxf(v, shfl_xor_f(v, off));
  return v;
}
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int off = SEG / 2; off >= 1; off >>= 1) v += shfl_xor_f(v, off);
  return v;
}

template <int SEG>
__global__ __launch_bounds__(256) void indexer_kl_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ block_idx,
    const float *__restrict__ block_mass, float *__restrict__ kl, float *__restrict__ grad, int K,
    int nb_max, int64_t total_q) {
  constexpr int RPW = 64 / SEG;  // rows per wave
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / SEG;
  const int slot = lane % SEG;
  const int g = blockIdx.y;
  // lanes of rows past the end (only in the last wave) and past k take part
  // in the reductions with neutral values
  const bool in = row < total_q && slot < K;
  const int64_t rk = ((int64_t)g * total_q + row) * K;
  const int j = in ? block_idx[rk + slot] : -1;
  const bool kept = j >= 0 && j < nb_max;
  const float sc = kept ? scores[((int64_t)g * total_q + row) * nb_max + j] : neg_inf();
  const float p = kept ? block_mass[rk + slot] : 0.f;
  const float M = seg_max<SEG>(sc);
  const bool live = kept && M != neg_inf();
  const float e = live ? expf(sc - M) : 0.f;
  const float Z = seg_sum<SEG>(e);
  const float P = seg_sum<SEG>(p);
  float klv = 0.f, gv = 0.f;
  if (live) {
    const float lnq = sc - M - logf(Z);
    klv = p > 0.f ? p * (logf(p) - lnq) : 0.f;
    gv = (e / Z) * P - p;
  }
  const float KL = seg_sum<SEG>(klv);
  if (in) grad[rk + slot] = gv;
  if (slot == 0 && row < total_q) kl[(int64_t)g * total_q + row] = KL;
}

}  // namespace

hipError_t launch_indexer_kl(const Dims &p, const float *scores, const int32_t *block_idx,
                             const float *block_mass, float *kl, float *grad, hipStream_t s) {
  if (p.total_q <= 0) return hipSuccess;
  const int seg = p.top_k <= 16 ? 16 : (p.top_k <= 32 ? 32 : 64);
  const int64_t rows_per_block = 4 * (64 / seg);
  const dim3 grid((unsigned)((p.total_q + rows_per_block - 1) / rows_per_block), (unsigned)p.G);
#define MSA_KL_CASE(S_)                                                                          \
  if (seg == S_)                                                                                 \
    hipLaunchKernelGGL(indexer_kl_kernel<S_>, grid, dim3(256), 0, s, scores, block_idx,         \
                       block_mass, kl, grad, p.top_k, p.nb_max, p.total_q);
  MSA_KL_CASE(16) MSA_KL_CASE(32) MSA_KL_CASE(64)
#undef MSA_KL_CASE
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace msa
