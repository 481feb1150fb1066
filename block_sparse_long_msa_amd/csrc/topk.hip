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
// stay in registers (NCH chunks of 64 per lane, up to 128).  Long rows first cut the
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
constexpr int kPruneMinChunks = 4;  // rows of fewer chunks go straight to the exact search

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

// One step of the bitwise search: keep `bit` in tau if at least `need` keys
// are >= tau | bit.  Bits HI..LO of the search, unrolled (no loop overhead on
// the scalar unit, which carries the counts).
template <int NC>
__device__ __forceinline__ uint32_t search_step(const uint32_t (&key)[NC], int need, uint32_t tau,
                                                uint32_t bit) {
  const uint32_t cand = tau | bit;
  int cnt = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) cnt += __popcll(ballot64(key[c] >= cand));
  return cnt >= need ? cand : tau;
}
template <int NC, int HI, int LO>
__device__ __forceinline__ uint32_t search_bits(const uint32_t (&key)[NC], int need, uint32_t tau) {
#pragma unroll
  for (int b = HI; b >= LO; --b) tau = search_step<NC>(key, need, tau, 1u << b);
  return tau;
}

// The need-th largest key when the answer is known to lie in [lo, hi] (at
// least `need` keys are >= lo and none is above hi), with bits below LOW left
// 0: for LOW > 0 the result is a lower bound that at least `need` keys still
// reach.  The answer shares the bits of lo and hi above their highest
// differing bit, so the search enters the unrolled bit sequence at bit 31, 23,
// 15 or 7, whichever is the first at or above that bit.
template <int NC, int LOW = 0>
__device__ __forceinline__ uint32_t kth_largest_in(const uint32_t (&key)[NC], int need, uint32_t lo,
                                                   uint32_t hi) {
  // lo and hi are wave-uniform: the search runs on scalar registers
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
  const uint32_t low_mask = ~((1u << LOW) - 1u);
  const uint32_t diff = lo ^ hi;
  if (diff < (1u << LOW)) return lo & low_mask;
  if (diff >= (1u << 24)) return search_bits<NC, 31, LOW>(key, need, 0u);
  if constexpr (LOW <= 23) {
    if (diff >= (1u << 16)) return search_bits<NC, 23, LOW>(key, need, lo & 0xff000000u);
  }
  if constexpr (LOW <= 15) {
    if (diff >= (1u << 8)) return search_bits<NC, 15, LOW>(key, need, lo & 0xffff0000u);
  }
  if constexpr (LOW <= 7) return search_bits<NC, 7, LOW>(key, need, lo & 0xffffff00u);
  return lo & low_mask;  // not reached: diff < 2^LOW was handled above
}

// Maximum key over the wave, wave-uniform.
template <int NC>
__device__ __forceinline__ uint32_t wave_max_key(const uint32_t (&key)[NC]) {
  uint32_t m = key[0];
#pragma unroll
  for (int c = 1; c < NC; ++c) m = max(m, key[c]);
  return wave_max_u32(m);
}

// A lower bound for the need-th largest of one value per lane (need <= 63):
// that value's top 16 bits, low bits 0.  At least `need` lanes are at or
// above it, and it is within 2^-7 (relative) of the exact value.
__device__ __forceinline__ uint32_t kth_largest_lanes_lb(uint32_t v, int need) {
  const uint32_t one[1] = {v};
  return kth_largest_in<1, 16>(one, need, wave_min_u32(v), wave_max_u32(v));
}

// Emits, in index order, every key > tau plus keys == tau while fewer than
// take_eq equal keys have been taken overall; eq_seen0 equal keys come
// before this wave's keys in index order, and the wave's first selected key
// goes to dst[out0].
template <int NC, typename IndexOf>
__device__ __forceinline__ void emit_from(const uint32_t (&key)[NC], IndexOf index_of,
                                          uint32_t tau, int take_eq, int out0, int eq_seen0,
                                          int32_t *dst) {
  int out_pos = out0, eq_seen = eq_seen0;
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

// Emits, in index order, every key > tau plus the first (need - #{> tau})
// keys == tau.  index_of(c) is the block index of key[c]; writes dst[0..need).
template <int NC, typename IndexOf>
__device__ __forceinline__ void emit_selected(const uint32_t (&key)[NC], IndexOf index_of,
                                              uint32_t tau, int need, int32_t *dst) {
  int gt = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) gt += __popcll(ballot64(key[c] > tau));
  emit_from<NC>(key, index_of, tau, need - gt, 0, 0, dst);
}

// LDS written and read back by lanes of the same wave: the wave's LDS
// operations complete in issue order; this keeps the compiler from moving
// them across each other.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave per (group, query row), four rows of one group per work-group
// (grid: query rows / 4 x groups).  Row, position and block index are
// wave-uniform scalars.  The row's candidate keys stay in registers: NCH
// chunks of 64 per lane, key j of the row in chunk j / 64, lane j % 64 (0 past
// the candidates: it ranks below every real key).
template <int NCH>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ scores,
                                                   int32_t *__restrict__ block_idx,
                                                   const int64_t *__restrict__ cu_q,
                                                   const int64_t *__restrict__ cu_kv,
                                                   int num_seqs, int64_t total_q,
                                                   int nb_max, int BS, int K) {
  __shared__ uint32_t cand_key_all[4][kCandCap];
  __shared__ int32_t cand_idx_all[4][kCandCap];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t *cand_key = cand_key_all[wave];
  int32_t *cand_idx = cand_idx_all[wave];
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= total_q) return;
  const int64_t grow = (int64_t)blockIdx.y * total_q + row;  // g * total_q + row
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  int32_t *dst = block_idx + grow * K;
  if (p < 0) {  // no causal key at all
    for (int i = lane; i < K; i += 64) dst[i] = -1;
    return;
  }
  const int J = (int)(p >> (31 - __builtin_clz(BS)));  // BS is a power of two
  const int need = K - 1;
  if (J <= need) {
    for (int i = lane; i < K; i += 64) dst[i] = i <= J ? i : -1;
    return;
  }
  const float *src = scores + grow * nb_max;
  // all chunks load at once: lanes past the candidates read block J - 1
  // (in the row) and take key 0
  uint32_t key[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int j = 64 * c + lane;
    key[c] = ordered_key(src[min(j, J - 1)]) & (j < J ? 0xffffffffu : 0u);
  }
  if (NCH >= kPruneMinChunks) {
    // Lower bound: the need-th largest of the group maxima (group r of a lane
    // = its chunks c with c % GPL == r; 64*GPL groups).  More than `need`
    // groups hold a candidate, so at least `need` keys are >= it; hence
    // every selected key, and every key tied with the last one, is >= it.
    // One group per lane leaves ~42 expected candidates for need = 31 on
    // i.i.d. scores, two per lane ~87 for need = 63.
    uint32_t lb;
    if (need <= 31) {
      uint32_t gmax = 0u;
#pragma unroll
      for (int c = 0; c < NCH; ++c) gmax = max(gmax, key[c]);
      lb = kth_largest_lanes_lb(gmax, need);
    } else {
      uint32_t gmax[2] = {0u, 0u};
#pragma unroll
      for (int c = 0; c < NCH; ++c) gmax[c & 1] = max(gmax[c & 1], key[c]);
      lb = kth_largest_in<2, 16>(gmax, need, wave_min_u32(min(gmax[0], gmax[1])),
                                 wave_max_u32(max(gmax[0], gmax[1])));
    }
    int n_cand = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) n_cand += __popcll(ballot64(key[c] >= lb));
    if (n_cand <= kCandCap) {
      int base = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const bool in = key[c] >= lb;
        const uint64_t m = ballot64(in);
        if (in) {
          cand_key[base + mbcnt64(m)] = key[c];
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
        const uint32_t tau = kth_largest_in<CC>(ck, need, lb, wave_max_key<CC>(ck));
        emit_selected<CC>(ck, [&](int c) { return ci[c]; }, tau, need, dst);
      };
      if (n_cand <= 64) finish(std::integral_constant<int, 1>());
      else if (n_cand <= 128) finish(std::integral_constant<int, 2>());
      else if (n_cand <= 256) finish(std::integral_constant<int, 4>());
      else finish(std::integral_constant<int, kCandCap / 64>());
      if (lane == 0) dst[need] = J;
      return;
    }
    // more keys tie at the bound than the candidate slice holds: exact
    // search over the whole row below
  }
  emit_selected<NCH>(key, [&](int c) { return 64 * c + lane; }, kth_largest<NCH>(key, need), need,
                     dst);
  if (lane == 0) dst[need] = J;
}

// Long rows (more than 2048 candidate blocks): one 4-wave work-group per
// row, wave w holding keys [w*64*NCW, (w+1)*64*NCW) in registers (NCW chunks
// of 64).  The waves share their lane maxima for the lower bound, compact
// their candidates at offsets given by the counts of the waves before them,
// so the list stays in index order, and wave 0 runs the exact search on the
// list.  If more keys tie at the bound than the list
// holds, the four waves run the bitwise search together and emit their keys
// at offsets given by the selected counts of the waves before them.
template <int NCW>
__global__ __launch_bounds__(256) void topk_long_kernel(const float *__restrict__ scores,
                                                        int32_t *__restrict__ block_idx,
                                                        const int64_t *__restrict__ cu_q,
                                                        const int64_t *__restrict__ cu_kv,
                                                        int num_seqs, int64_t total_q, int nb_max,
                                                        int BS, int K) {
  __shared__ uint32_t gmax_sh[4 * 64];
  __shared__ int cnt_sh[2][4];
  __shared__ uint32_t cand_key[kCandCap];
  __shared__ int32_t cand_idx[kCandCap];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = blockIdx.x;
  const int64_t grow = (int64_t)blockIdx.y * total_q + row;  // g * total_q + row
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  int32_t *dst = block_idx + grow * K;
  if (p < 0) {
    for (int i = threadIdx.x; i < K; i += 256) dst[i] = -1;
    return;
  }
  const int J = (int)(p >> (31 - __builtin_clz(BS)));  // BS is a power of two
  const int need = K - 1;
  if (J <= need) {
    for (int i = threadIdx.x; i < K; i += 256) dst[i] = i <= J ? i : -1;
    return;
  }
  const float *src = scores + grow * nb_max;
  const int j0 = wave * 64 * NCW;
  uint32_t key[NCW];
#pragma unroll
  for (int c = 0; c < NCW; ++c) {
    const int j = j0 + 64 * c + lane;
    key[c] = ordered_key(src[min(j, J - 1)]) & (j < J ? 0xffffffffu : 0u);
  }
  // Lower bound: the need-th largest of the maxima of the 64 residue classes
  // j mod 64 (lane l of every wave holds class l).  The first J keys fall in
  // min(J, 64) > need classes, so at least `need` keys are >= it.
  uint32_t gm = 0u;
#pragma unroll
  for (int c = 0; c < NCW; ++c) gm = max(gm, key[c]);
  gmax_sh[wave * 64 + lane] = gm;
  __syncthreads();
  const uint32_t cls = max(max(gmax_sh[lane], gmax_sh[64 + lane]),
                           max(gmax_sh[128 + lane], gmax_sh[192 + lane]));
  const uint32_t lb = kth_largest_lanes_lb(cls, need);
  int n = 0;
#pragma unroll
  for (int c = 0; c < NCW; ++c) n += __popcll(ballot64(key[c] >= lb));
  if (lane == 0) cnt_sh[0][wave] = n;
  __syncthreads();
  int total = 0, off = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int cw = cnt_sh[0][w];
    off += w < wave ? cw : 0;
    total += cw;
  }
  if (total <= kCandCap) {
    int base = off;
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      const bool in = key[c] >= lb;
      const uint64_t m = ballot64(in);
      if (in) {
        cand_key[base + mbcnt64(m)] = key[c];
        cand_idx[base + mbcnt64(m)] = j0 + 64 * c + lane;
      }
      base += __popcll(m);
    }
    __syncthreads();
    if (wave != 0) return;
    auto finish = [&](auto tag) {
      constexpr int CC = decltype(tag)::value;
      uint32_t ck[CC];
      int ci[CC];
#pragma unroll
      for (int c = 0; c < CC; ++c) {
        const int i = 64 * c + lane;
        ck[c] = i < total ? cand_key[i] : 0u;
        ci[c] = i < total ? cand_idx[i] : 0;
      }
      const uint32_t tau = kth_largest_in<CC>(ck, need, lb, wave_max_key<CC>(ck));
      emit_selected<CC>(ck, [&](int c) { return ci[c]; }, tau, need, dst);
    };
    if (total <= 64) finish(std::integral_constant<int, 1>());
    else if (total <= 128) finish(std::integral_constant<int, 2>());
    else if (total <= 256) finish(std::integral_constant<int, 4>());
    else finish(std::integral_constant<int, kCandCap / 64>());
    if (lane == 0) dst[need] = J;
    return;
  }
  // Cooperative exact search: bit by bit, the four waves' counts are summed
  // through LDS (two count slots alternate, so one barrier per bit is enough).
  uint32_t tau = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < NCW; ++c) cnt += __popcll(ballot64(key[c] >= cand));
    if (lane == 0) cnt_sh[bit & 1][wave] = cnt;
    __syncthreads();
    const int tot = cnt_sh[bit & 1][0] + cnt_sh[bit & 1][1] + cnt_sh[bit & 1][2] + cnt_sh[bit & 1][3];
    if (tot >= need) tau = cand;
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int c = 0; c < NCW; ++c) {
    gt += __popcll(ballot64(key[c] > tau));
    eq += __popcll(ballot64(key[c] == tau));
  }
  __syncthreads();  // every wave is done reading the count slots
  if (lane == 0) {
    cnt_sh[0][wave] = gt;
    cnt_sh[1][wave] = eq;
  }
  __syncthreads();
  int GT = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) GT += cnt_sh[0][w];
  const int take_eq = need - GT;
  int out0 = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    const int e = cnt_sh[1][w];
    out0 += cnt_sh[0][w] + min(max(take_eq - eq_before, 0), e);
    eq_before += e;
  }
  emit_from<NCW>(key, [&](int c) { return j0 + 64 * c + lane; }, tau, take_eq, out0, eq_before,
                 dst);
  if (threadIdx.x == 0) dst[need] = J;
}

template <int NCW>
hipError_t launch_long(const Dims &p, const float *scores, int32_t *block_idx, hipStream_t s) {
  hipLaunchKernelGGL((topk_long_kernel<NCW>), dim3((unsigned)p.total_q, p.G), dim3(256), 0, s, scores,
                     block_idx, p.cu_q, p.cu_kv, p.num_seqs, p.total_q, p.nb_max, p.B, p.top_k);
  profile_mark(s);
  return hipGetLastError();
}

template <int NCH>
hipError_t launch_nch(const Dims &p, const float *scores, int32_t *block_idx, hipStream_t s) {
  dim3 grid((unsigned)((p.total_q + 3) / 4), p.G);
  hipLaunchKernelGGL((topk_kernel<NCH>), grid, dim3(256), 0, s, scores, block_idx, p.cu_q,
                     p.cu_kv, p.num_seqs, p.total_q, p.nb_max, p.B, p.top_k);
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
  if (nch <= 32) return launch_nch<32>(p, scores, block_idx, s);
  // rows of up to 4096 / 8192 blocks: four waves per row
  if (nch <= 64) return launch_long<16>(p, scores, block_idx, s);
  if (nch <= 128) return launch_long<32>(p, scores, block_idx, s);
  return hipErrorInvalidValue;  // rows are at most 8192 blocks (checked at the API)
}

}  // namespace msa
