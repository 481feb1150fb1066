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
// stay in registers (NCH chunks of 64 per lane).  Long rows first cut the
// search down: the (k-1)-th largest of the 64 lane maxima (128 half-lane
// maxima when k-1 > 31) is a lower bound of the answer, and the few keys at
// or above it (kept in index order in LDS) hold every selected key; the
// exact search then runs on those only.
#include <type_traits>

#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kCandCap = 512;  // candidates kept for the exact search (8 per lane)
constexpr int kPruneMinChunks = 8;  // rows of fewer chunks go straight to the exact search

// Exact need-th largest key among NC chunks of 64 keys (0 = absent).
template <int NC>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&key)[NC], int need) {
  uint32_t tau = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) cnt += __popcll(ballot64(key[c] >= cand));
    if (cnt >= need) tau = cand;
  }
  return tau;
}

// Emits, in index order, every key > tau plus the first (need - #{> tau})
// keys == tau.  index_of(c) is the block index of key[c]; writes dst[0..need).
template <int NC, typename IndexOf>
__device__ __forceinline__ void emit_selected(const uint32_t (&key)[NC], IndexOf index_of,
                                              uint32_t tau, int need, int32_t *dst) {
  int gt = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) gt += __popcll(ballot64(key[c] > tau));
  const int take_eq = need - gt;
  int out_pos = 0, eq_seen = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const bool is_gt = key[c] > tau, is_eq = key[c] == tau;
    const uint64_t eqm = ballot64(is_eq);
    const bool sel = is_gt || (is_eq && eq_seen + mbcnt64(eqm) < take_eq);
    const uint64_t selm = ballot64(sel);
    if (sel) dst[out_pos + mbcnt64(selm)] = index_of(c);
    out_pos += __popcll(selm);
    eq_seen += __popcll(eqm);
  }
}

// LDS written and read back by lanes of the same wave: the wave's LDS
// operations complete in issue order; this keeps the compiler from moving
// them across each other.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave per (group, query row), four rows per work-group.  NCH > 0: the
// row's keys stay in registers (NCH chunks of 64 per lane).  NCH == 0: long
// rows; keys are streamed from the score row (L2-resident after one pass).
template <int NCH>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ scores,
                                                   int32_t *__restrict__ block_idx,
                                                   const int64_t *__restrict__ cu_q,
                                                   const int64_t *__restrict__ cu_kv,
                                                   int num_seqs, int G, int64_t total_q,
                                                   int nb_max, int BS, int K) {
  __shared__ uint32_t cand_key_all[4][kCandCap];
  __shared__ int32_t cand_idx_all[4][kCandCap];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t *cand_key = cand_key_all[wave];
  int32_t *cand_idx = cand_idx_all[wave];
  const int64_t grow = (int64_t)blockIdx.x * 4 + wave;  // g * total_q + row
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
  const int nch = (J + 63) / 64;  // chunks holding candidates
  constexpr int R = NCH > 0 ? NCH : 1;
  uint32_t key[R];
  auto key_at = [&](int c) -> uint32_t {  // c < nch
    if (NCH > 0) return key[c];
    const int j = 64 * c + lane;
    return j < J ? ordered_key(src[j]) : 0u;
  };
  if (NCH > 0) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int j = 64 * c + lane;
      key[c] = j < J ? ordered_key(src[j]) : 0u;  // 0 ranks below every real key
    }
  }
  if (NCH == 0 || NCH >= kPruneMinChunks) {
    // Lower bound: the need-th largest of the group maxima (group r of a lane
    // = its chunks c with c % GPL == r; 64*GPL groups).  More than `need`
    // groups hold a candidate, so at least `need` keys are >= it; hence
    // every selected key, and every key tied with the last one, is >= it.
    // One group per lane leaves ~42 expected candidates for need = 31 on
    // i.i.d. scores, two per lane ~87 for need = 63.
    uint32_t lb;
    if (need <= 31) {
      uint32_t gmax[1] = {0u};
      for (int c = 0; c < nch; ++c) gmax[0] = max(gmax[0], key_at(c));
      lb = kth_largest<1>(gmax, need);
    } else {
      uint32_t gmax[2] = {0u, 0u};
      for (int c = 0; c < nch; ++c) gmax[c & 1] = max(gmax[c & 1], key_at(c));
      lb = kth_largest<2>(gmax, need);
    }
    int n_cand = 0;
    for (int c = 0; c < nch; ++c) n_cand += __popcll(ballot64(key_at(c) >= lb));
    if (n_cand <= kCandCap) {
      int base = 0;
      for (int c = 0; c < nch; ++c) {
        const uint32_t kc = key_at(c);
        const bool in = kc >= lb;
        const uint64_t m = ballot64(in);
        if (in) {
          cand_key[base + mbcnt64(m)] = kc;
          cand_idx[base + mbcnt64(m)] = 64 * c + lane;
        }
        base += __popcll(m);
      }
      wave_lds_sync();
      auto finish = [&](auto tag) {
        constexpr int CC = decltype(tag)::value;
        uint32_t ck[CC];
        int ci[CC];
#pragma unroll
        for (int c = 0; c < CC; ++c) {
          const int i = 64 * c + lane;
          ck[c] = i < n_cand ? cand_key[i] : 0u;
          ci[c] = i < n_cand ? cand_idx[i] : 0;
        }
        emit_selected<CC>(ck, [&](int c) { return ci[c]; }, kth_largest<CC>(ck, need), need, dst);
      };
      if (n_cand <= 128) finish(std::integral_constant<int, 2>());
      else finish(std::integral_constant<int, kCandCap / 64>());
      if (lane == 0) dst[need] = J;
      return;
    }
  }
  if (NCH > 0) {
    emit_selected<R>(key, [&](int c) { return 64 * c + lane; }, kth_largest<R>(key, need), need,
                     dst);
  } else {
    // Too many keys tie at the lower bound: exact search with streamed keys.
    uint32_t tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int cnt = 0;
      for (int c = 0; c < nch; ++c) cnt += __popcll(ballot64(key_at(c) >= cand));
      if (cnt >= need) tau = cand;
    }
    int gt = 0;
    for (int c = 0; c < nch; ++c) gt += __popcll(ballot64(key_at(c) > tau));
    const int take_eq = need - gt;
    int out_pos = 0, eq_seen = 0;
    for (int c = 0; c < nch; ++c) {
      const uint32_t kc = key_at(c);
      const bool is_gt = kc > tau, is_eq = kc == tau;
      const uint64_t eqm = ballot64(is_eq);
      const bool sel = is_gt || (is_eq && eq_seen + mbcnt64(eqm) < take_eq);
      const uint64_t selm = ballot64(sel);
      if (sel) dst[out_pos + mbcnt64(selm)] = 64 * c + lane;
      out_pos += __popcll(selm);
      eq_seen += __popcll(eqm);
    }
  }
  if (lane == 0) dst[need] = J;
}

template <int NCH>
hipError_t launch_nch(const Dims &p, const float *scores, int32_t *block_idx, hipStream_t s) {
  const int64_t rows = (int64_t)p.G * p.total_q;
  dim3 grid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL((topk_kernel<NCH>), grid, dim3(256), 0, s, scores, block_idx, p.cu_q,
                     p.cu_kv, p.num_seqs, p.G, p.total_q, p.nb_max, p.B, p.top_k);
  profile_mark(s);
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
  return launch_nch<0>(p, scores, block_idx, s);  // long rows: streamed keys
}

}  // namespace msa
