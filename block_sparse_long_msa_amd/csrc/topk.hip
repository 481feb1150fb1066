// Per-group Top-k block selection with the current block always kept
// ("MiniMax Sparse Attention" page, Summary, paragraph 2; k counts the kept
// current block, as the Key points "Benchmark configuration" bullet's
// 16 x 128 = 2,048 attended tokens shows).
//
// One wave per (group, query row).  For a row at position p the current
// block is J = p / B and the candidates are blocks 0..J-1.  If J <= k-1 every
// causal block is kept.  Otherwise the (k-1)-th largest candidate score is
// found exactly by a 32-step bitwise search over order-preserving uint32 keys
// (comparisons and ballot counts only - no exponentials), then the kept set
// is every key above it plus the lowest-index keys equal to it.  Scanning the
// candidates in index order with ballot prefix counts emits them ascending;
// J (larger than every candidate) comes last.  The candidate keys of a row
// stay in registers (NCH chunks of 64 per lane).
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

template <int NCH>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ scores,
                                                   int32_t *__restrict__ block_idx,
                                                   const int64_t *__restrict__ cu_q,
                                                   const int64_t *__restrict__ cu_kv,
                                                   int num_seqs, int G, int64_t total_q,
                                                   int nb_max, int BS, int K) {
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // g * total_q + row
  if (grow >= (int64_t)G * total_q) return;
  const int64_t row = grow % total_q;
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  int32_t *dst = block_idx + grow * K;
  if (p < 0) {  // no causal key at all
    for (int i = lane; i < K; i += 64) dst[i] = -1;
    return;
  }
  const int J = (int)(p / BS);
  const int need = K - 1;
  if (J <= need) {
    for (int i = lane; i < K; i += 64) dst[i] = i <= J ? i : -1;
    return;
  }
  const float *src = scores + grow * nb_max;
  uint32_t key[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int j = 64 * c + lane;
    key[c] = j < J ? ordered_key(src[j]) : 0u;  // 0 ranks below every real key
  }
  // tau = largest x with #{key >= x} >= need, i.e. the need-th largest key.
  uint32_t tau = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) cnt += __popcll(ballot64(key[c] >= cand));
    if (cnt >= need) tau = cand;
  }
  int gt = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) gt += __popcll(ballot64(key[c] > tau));
  const int take_eq = need - gt;  // >= 1
  int out_pos = 0, eq_seen = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const bool is_gt = key[c] > tau, is_eq = key[c] == tau;
    const uint64_t eqm = ballot64(is_eq);
    const bool sel = is_gt || (is_eq && eq_seen + mbcnt64(eqm) < take_eq);
    const uint64_t selm = ballot64(sel);
    if (sel) dst[out_pos + mbcnt64(selm)] = 64 * c + lane;
    out_pos += __popcll(selm);
    eq_seen += __popcll(eqm);
  }
  if (lane == 0) dst[need] = J;
}

template <int NCH>
hipError_t launch_nch(const Dims &p, const float *scores, int32_t *block_idx, hipStream_t s) {
  const int64_t rows = (int64_t)p.G * p.total_q;
  dim3 grid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL((topk_kernel<NCH>), grid, dim3(256), 0, s, scores, block_idx, p.cu_q,
                     p.cu_kv, p.num_seqs, p.G, p.total_q, p.nb_max, p.B, p.top_k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const Dims &p, const float *scores, int32_t *block_idx, hipStream_t s) {
  if (p.total_q <= 0) return hipSuccess;
  const int nch = (p.nb_max + 63) / 64;
  if (nch <= 1) return launch_nch<1>(p, scores, block_idx, s);
  if (nch <= 2) return launch_nch<2>(p, scores, block_idx, s);
  if (nch <= 4) return launch_nch<4>(p, scores, block_idx, s);
  if (nch <= 8) return launch_nch<8>(p, scores, block_idx, s);
  if (nch <= 16) return launch_nch<16>(p, scores, block_idx, s);
  if (nch <= 32) return launch_nch<32>(p, scores, block_idx, s);
  if (nch <= 64) return launch_nch<64>(p, scores, block_idx, s);
  if (nch <= 128) return launch_nch<128>(p, scores, block_idx, s);
  return hipErrorInvalidValue;
}

}  // namespace msa
