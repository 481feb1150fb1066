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
// One wave per (group, row), one lane per slot (k <= 64); four rows of one
// group per work-group.  The work is k gathered scores and k masses per row:
// a small, latency-bound kernel next to the forward pass.
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, shfl_xor_f(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += shfl_xor_f(v, off);
  return v;
}

__global__ __launch_bounds__(256) void indexer_kl_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ block_idx,
    const float *__restrict__ block_mass, float *__restrict__ kl, float *__restrict__ grad, int K,
    int nb_max, int64_t total_q) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= total_q) return;  // the whole wave leaves together
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t rk = ((int64_t)g * total_q + row) * K;
  const bool in = lane < K;
  const int j = in ? block_idx[rk + lane] : -1;
  const bool kept = j >= 0 && j < nb_max;
  const float sc = kept ? scores[((int64_t)g * total_q + row) * nb_max + j] : neg_inf();
  const float p = kept ? block_mass[rk + lane] : 0.f;
  const float M = wave_max_f(sc);
  const bool live = kept && M != neg_inf();
  const float e = live ? expf(sc - M) : 0.f;
  const float Z = wave_sum_f(e);
  const float P = wave_sum_f(p);
  float klv = 0.f, gv = 0.f;
  if (live) {
    const float lnq = sc - M - logf(Z);
    klv = p > 0.f ? p * (logf(p) - lnq) : 0.f;
    gv = (e / Z) * P - p;
  }
  const float KL = wave_sum_f(klv);
  if (in) grad[rk + lane] = gv;
  if (lane == 0) kl[(int64_t)g * total_q + row] = KL;
}

}  // namespace

hipError_t launch_indexer_kl(const Dims &p, const float *scores, const int32_t *block_idx,
                             const float *block_mass, float *kl, float *grad, hipStream_t s) {
  if (p.total_q <= 0) return hipSuccess;
  const dim3 grid((unsigned)((p.total_q + 3) / 4), (unsigned)p.G);
  hipLaunchKernelGGL(indexer_kl_kernel, grid, dim3(256), 0, s, scores, block_idx, block_mass, kl,
                     grad, p.top_k, p.nb_max, p.total_q);
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace msa
