// Index Branch scoring fused with the Top-k selection ("MiniMax Sparse
// Attention" page, Summary paragraphs 2 and 3: max-pooled block scores, a
// per-group Top-k with the current block kept, selected by comparisons only),
// without materialising the [G, total_q, NBmax] score tensor.
//
// Two kernels:
//  * index_topk_kernel - a work-group (8 waves, 64 queries each) owns a tile
//    of 512 queries of one (sequence, group) and a segment of key blocks.  It
//    streams the segment's index-key blocks through a two-stage LDS ring
//    (direct global-to-LDS loads, XOR-swizzled 16-byte chunks), computes each
//    block's max-pooled score with the same 32x32x16 bf16 MFMA chain and max
//    as msa_index_score (so every score is bit-identical to it), and keeps,
//    per query, the best candidate blocks seen so far in a sorted list in
//    registers (at least k-1 of them).  Candidates are the blocks below the
//    query's current block J, which are wholly causal, so no mask is needed;
//    J itself is forced and blocks past it are never candidates.  Blocks
//    arrive in ascending order, so ranking by score alone and placing a new
//    block after every entry of equal score gives (score descending, block
//    ascending) exactly.  At the end of the segment the list goes to the
//    workspace as 64-bit keys ordered(score) << 32 | (2^32 - 1 - block): a
//    larger key is a better candidate.
//  * index_topk_merge_kernel - one wave per (group, row): the k-1 largest
//    keys over the row's segments (all keys are distinct), then listed in
//    ascending block order with J appended and -1 padding; rows with
//    J <= k-1 keep 0..J without any score.
#include <algorithm>

#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

// Index-key block of BS rows x DI bf16: 16-byte chunks XOR-swizzled so that
// the 32 rows read by one MFMA operand load hit distinct LDS banks.
template <int DI, int BS>
struct FusedTile {
  static constexpr int CPR = DI / 8;        // 16-byte chunks per key row
  static constexpr int CHUNKS = BS * CPR;   // chunks per block
  static constexpr int STAGE = CHUNKS * 16; // bytes per staged block
  static constexpr int RPB = 16 / CPR;      // rows sharing one 64-bank line
  __device__ static __forceinline__ int swz(int r, int q) { return r * CPR + (q ^ ((r / RPB) % CPR)); }
};

__device__ __forceinline__ void dma16_fused(const uint16_t *src, uint8_t *lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)lds, 16, 0, 0);
}

// Inserts candidate (nk, nj) into a lane's list of the CAPP best candidates,
// held in registers in descending key order (key = ordered score, 0 = empty).
// Blocks arrive in ascending order, so a new candidate ranks after every
// entry whose score is greater or equal (those have lower block indices): it
// goes in at the first position whose key it beats strictly, and the entries
// from there on move down one place (the last drops out).  Branchless: every
// lane runs the same compare-and-select network.
template <int CAPP>
__device__ __forceinline__ void list_insert(uint32_t (&key)[CAPP], uint32_t (&blk)[CAPP],
                                            uint32_t nk, uint32_t nj) {
  uint32_t ck = nk, cj = nj;  // the value carried down the list
#pragma unroll
  for (int i = 0; i < CAPP; ++i) {
    const bool here = ck > key[i];       // carried value goes in at i, old entry i carries on
    const uint32_t k_old = key[i], j_old = blk[i];
    key[i] = here ? ck : k_old;
    blk[i] = here ? cj : j_old;
    ck = here ? k_old : ck;
    cj = here ? j_old : cj;
  }
}

template <int DI, int BS, int CAPP>
__global__ __launch_bounds__(512) void index_topk_kernel(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    uint64_t *__restrict__ cand, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int G, int64_t total_q, int nqt, int nbg, int seg,
    int nseg) {
  using T = FusedTile<DI, BS>;
  constexpr int NW = 8;
  constexpr int QT = 64 * NW;     // queries per work-group
  constexpr int KT = BS / 32;     // 32-key tiles per block
  constexpr int NK = DI / 16;     // MFMA steps over d_idx
  constexpr int NLD = T::CHUNKS / 64;          // 64-lane direct loads per block
  constexpr int LPW = (NLD + NW - 1) / NW;     // of them per wave
  static_assert(T::CHUNKS % 64 == 0, "whole 64-slot loads");
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  // Work-group order: segment-major, then (sequence, group), then query tiles
  // from the last (longest rows) to the first.  Consecutive work-groups share
  // a segment's index keys; the round-robin deal to the XCDs runs tiles of
  // one segment on every XCD at once.
  int local = blockIdx.x;
  const int qt = nqt - 1 - local % nqt;
  local /= nqt;
  const int bg = local % nbg;          // sequence * G + group
  const int s_id = local / nbg;        // segment
  const int b = bg / G, g = bg - b * G;
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t t0 = (int64_t)qt * QT;
  if (t0 >= sq.lq) return;
  const int nq = (int)min<int64_t>(QT, sq.lq - t0);
  const int64_t p_last = sq.base + t0 + nq - 1;
  if (p_last < 0) return;
  const int J_last = (int)(p_last / BS);
  const int js = s_id * seg;
  const int je = min(js + seg, J_last);  // candidate blocks of the tile lie below J_last
  if (je <= js) return;                  // no row of the tile has a candidate here

  const int q = wave * 64 + lane;              // this lane's query column after the max
  const int64_t pos = sq.base + t0 + q;
  const int Jq = (q < nq && pos >= 0) ? (int)(pos / BS) : 0;
  uint32_t lkey[CAPP], lblk[CAPP];
#pragma unroll
  for (int i = 0; i < CAPP; ++i) {
    lkey[i] = 0;
    lblk[i] = 0;
  }

  // index queries of the two 32-column halves as MFMA B operands
  bf16x8 qb[2][NK];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qn = wave * 64 + s * 32 + col;
    if (qn < nq) {
      const uint16_t *src = q_idx + ((sq.q0 + t0 + qn) * G + g) * (int64_t)DI + 8 * half;
#pragma unroll
      for (int c = 0; c < NK; ++c) qb[s][c] = as_bf16x8(ld16(src + 16 * c));
    } else {
#pragma unroll
      for (int c = 0; c < NK; ++c) qb[s][c] = zero_bf16x8();
    }
  }

  // Direct loads: load L of a block fills slots [64L, 64L + 64); wave w
  // issues loads w, w + NW, ...; lane l fetches the chunk the swizzle puts in
  // slot 64L + l.  Every block below J_last is complete in memory.
  const int64_t kstride = (int64_t)G * DI;
  const uint16_t *kbase = k_idx + ((sq.kv0 + (int64_t)js * BS) * G + g) * (int64_t)DI;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint16_t *kdma[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int S = min(64 * (wave_u + NW * i) + lane, T::CHUNKS - 1);
    const int r = S / T::CPR;
    kdma[i] = kbase + r * kstride + 8 * ((S % T::CPR) ^ ((r / T::RPB) % T::CPR));
  }
  const int64_t kblock = (int64_t)BS * kstride;
  auto dma = [&](int it, uint8_t *dst) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int L = wave_u + NW * i;
      if (NLD % NW != 0 && L >= NLD) break;
      dma16_fused(kdma[i] + it * kblock, dst + 1024 * L);
    }
  };
  // One block: the max over its keys of every query of the wave (the same
  // MFMA chain as msa_index_score), then, if some lane's query admits it,
  // the insertion network.
  auto block = [&](int it, const uint8_t *cur) {
    float m0 = neg_inf(), m1 = neg_inf();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      u32x4 kf[NK];
      const int r = kt * 32 + col;
#pragma unroll
      for (int c = 0; c < NK; ++c)
        kf[c] = *reinterpret_cast<const u32x4 *>(cur + 16 * T::swz(r, 2 * c + half));
      f32x16 a0 = {}, a1 = {};
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        a0 = mfma32x32x16(as_bf16x8(kf[c]), qb[0][c], a0);
        a1 = mfma32x32x16(as_bf16x8(kf[c]), qb[1][c], a1);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        m0 = fmaxf(m0, a0[e]);
        m1 = fmaxf(m1, a1[e]);
      }
    }
    const float m = halves_max_f(m0, m1);
    const int j = js + it;
    const uint32_t key = ordered_key(m);
    const bool admit = q < nq && j < Jq && key > lkey[CAPP - 1];
    if (ballot64(admit) != 0) {
      // lanes that do not admit insert a key of 0, which changes nothing
      list_insert<CAPP>(lkey, lblk, admit ? key : 0u, (uint32_t)j);
    }
  };
  const int nblk = je - js;
  dma(0, stage0);
  for (int it = 0; it < nblk; it += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block it in stage0; every wave is done with stage1
    if (it + 1 < nblk) dma(it + 1, stage1);
    block(it, stage0);
    if (it + 1 < nblk) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // block it+1 in stage1; every wave is done with stage0
      if (it + 2 < nblk) dma(it + 2, stage0);
      block(it + 1, stage1);
    }
  }
  // the list of every row that has a candidate in this segment, as 64-bit
  // keys ordered(score) << 32 | (2^32 - 1 - block) (0 where empty)
  if (q < nq && Jq > js) {
    uint64_t *dst = cand + (((int64_t)g * total_q + sq.q0 + t0 + q) * nseg + s_id) * CAPP;
#pragma unroll
    for (int i = 0; i < CAPP; i += 2) {
      const uint64_t a = lkey[i] == 0 ? 0 : ((uint64_t)lkey[i] << 32) | (0xFFFFFFFFu - lblk[i]);
      const uint64_t c = lkey[i + 1] == 0 ? 0 : ((uint64_t)lkey[i + 1] << 32) | (0xFFFFFFFFu - lblk[i + 1]);
      *reinterpret_cast<u32x4 *>(dst + i) =
          u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)c, (uint32_t)(c >> 32)};
    }
  }
}

// Count over a wave's live candidate slots of those satisfying `pred`.
template <int MAXS, typename F>
__device__ __forceinline__ int wave_count(int live, F pred) {
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < MAXS; ++u)
    if (u < live) cnt += __popcll(ballot64(pred(u)));
  return cnt;
}

// One wave per (group, row); four rows of one group per work-group.  The
// row's candidates are the lists of its segments (lst 64-bit keys each, 0
// where empty).  The kept K - 1 are the largest keys: first the (K-1)-th
// largest score key tau (a bitwise search over its 32 bits with ballot
// counts), then, if more candidates tie at tau than places remain, the
// lowest blocks among them (a second search over the low words, which hold
// 2^32 - 1 - block).
__global__ __launch_bounds__(256) void index_topk_merge_kernel(
    const uint64_t *__restrict__ cand, int32_t *__restrict__ block_idx,
    const int64_t *__restrict__ cu_q, const int64_t *__restrict__ cu_kv, int num_seqs, int BS,
    int K, int nseg, int seg, int lst, int64_t total_q) {
  constexpr int MAXS = 16;  // candidate slots per lane: 64 * 16 >= nseg * lst
  __shared__ int32_t sel[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= total_q) return;
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  int32_t *out = block_idx + ((int64_t)g * total_q + row) * K;
  if (p < 0) {
    if (lane < K) out[lane] = -1;
    return;
  }
  const int J = (int)(p / BS);
  if (J <= K - 1) {
    if (lane < K) out[lane] = lane <= J ? lane : -1;
    return;
  }
  if (K == 1) {  // only the current block; no candidate lists exist (no workspace)
    if (lane == 0) out[0] = J;
    return;
  }
  const int cap = K - 1;
  const int ns = (J + seg - 1) / seg;  // segments holding candidates of this row
  const int n = ns * lst;
  const int live = (n + 63) >> 6;      // slots in use (wave-uniform)
  MSA_DCHECK(ns <= nseg && n <= 64 * MAXS);
  const uint64_t *src = cand + ((int64_t)g * total_q + row) * nseg * lst;
  uint32_t hi[MAXS], lo[MAXS];
#pragma unroll
  for (int u = 0; u < MAXS; ++u) {
    const int i = lane + 64 * u;
    const uint64_t v = (u < live && i < n) ? src[i] : 0;
    hi[u] = (uint32_t)(v >> 32);
    lo[u] = (uint32_t)v;
  }
  // tau: the largest t with #{hi >= t} >= cap (every real candidate has
  // hi > 0, and the row has at least cap of them: J > cap candidates, each
  // segment keeping min(lst, its candidates))
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = tau | (1u << bit);
    if (wave_count<MAXS>(live, [&](int u) { return hi[u] >= t; }) >= cap) tau = t;
  }
  const int c_gt = tau == 0xFFFFFFFFu ? 0 : wave_count<MAXS>(live, [&](int u) { return hi[u] > tau; });
  const int need = cap - c_gt;  // candidates to take among those tied at tau
  const int c_eq = wave_count<MAXS>(live, [&](int u) { return hi[u] == tau; });
  uint32_t lo_min = 0;          // take the tied ones with lo >= lo_min
  if (c_eq > need) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = lo_min | (1u << bit);
      if (wave_count<MAXS>(live, [&](int u) { return hi[u] == tau && lo[u] >= t; }) >= need)
        lo_min = t;
    }
  }
  // list the K - 1 selected blocks (ballot prefix order), then place each by
  // its rank among them: ascending block order
  int base = 0;
#pragma unroll
  for (int u = 0; u < MAXS; ++u) {
    if (u >= live) break;
    const bool take = hi[u] > tau || (hi[u] == tau && lo[u] >= lo_min);
    const uint64_t m = ballot64(take);
    MSA_DCHECK(!take || base + (int)mbcnt64(m) < cap);
    if (take) sel[wv][base + mbcnt64(m)] = (int32_t)(0xFFFFFFFFu - lo[u]);
    base += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < cap) {
    const int32_t mine = sel[wv][lane];
    int rank = 0;
    for (int i = 0; i < cap; ++i) rank += sel[wv][i] < mine;
    MSA_DCHECK(mine >= 0 && mine < J);
    out[rank] = mine;
  }
  if (lane == 0) out[cap] = J;
}

template <int DI, int BS, int CAPP>
hipError_t launch_fused(const Dims &p, const uint16_t *q_idx, const uint16_t *k_idx,
                        uint64_t *cand, int nseg, int seg, hipStream_t s) {
  constexpr int QT = 512;
  const int nqt = (p.max_q_len + QT - 1) / QT;
  const int nbg = p.num_seqs * p.G;
  const int64_t nwg = (int64_t)nseg * nqt * nbg;
  if (nwg > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((index_topk_kernel<DI, BS, CAPP>), dim3((unsigned)nwg), dim3(512), 0, s,
                     q_idx, k_idx, cand, p.cu_q, p.cu_kv, p.G, p.total_q, nqt, nbg, seg, nseg);
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace

MSA_DEBUG_COUNTER(index_topk)

// Candidates kept per (query, segment): k - 1 rounded up to a power of two
// (at least 4), so the list's compare-and-select network is unrolled for a
// few sizes only; a longer list only keeps more candidates.
int index_topk_list(const Dims &p) {
  if (p.top_k <= 1) return 0;  // only the current block is kept: nothing to rank
  int c = 4;
  while (c < p.top_k - 1) c *= 2;
  return c;
}
// Segment length: 8 list lengths of key blocks, so a segment's candidates
// take a quarter of the bytes of its scores.
int index_topk_segment(const Dims &p) { return 8 * std::max(4, index_topk_list(p)); }
int index_topk_nseg(const Dims &p) {
  const int seg = index_topk_segment(p);
  return std::max(1, (p.nb_max + seg - 1) / seg);
}
size_t index_topk_workspace_bytes(const Dims &p) {
  if (p.top_k <= 1 || p.total_q == 0) return 0;
  return sizeof(uint64_t) * (size_t)p.G * (size_t)p.total_q * (size_t)index_topk_nseg(p) *
         (size_t)index_topk_list(p);
}
bool index_topk_supported(const Dims &p) {
  // the merge holds a row's candidates in 16 slots per lane
  return (int64_t)index_topk_nseg(p) * index_topk_list(p) <= 64 * 16;
}

hipError_t launch_index_topk(const Dims &p, const uint16_t *q_idx, const uint16_t *k_idx,
                             int32_t *block_idx, void *workspace, hipStream_t s) {
  if (p.total_q <= 0) return hipSuccess;
  const int seg = index_topk_segment(p);
  const int nseg = index_topk_nseg(p);
  const int lst = index_topk_list(p);
  uint64_t *cand = static_cast<uint64_t *>(workspace);
  if (p.top_k > 1 && p.nb_max > 1) {
    hipError_t e = hipErrorInvalidValue;
#define MSA_FUSED_CASE(DI_, BS_)                                                         \
  if (p.d_idx == DI_ && p.B == BS_) {                                                   \
    if (lst == 4) e = launch_fused<DI_, BS_, 4>(p, q_idx, k_idx, cand, nseg, seg, s);   \
    else if (lst == 8) e = launch_fused<DI_, BS_, 8>(p, q_idx, k_idx, cand, nseg, seg, s); \
    else if (lst == 16) e = launch_fused<DI_, BS_, 16>(p, q_idx, k_idx, cand, nseg, seg, s); \
    else if (lst == 32) e = launch_fused<DI_, BS_, 32>(p, q_idx, k_idx, cand, nseg, seg, s); \
    else e = launch_fused<DI_, BS_, 64>(p, q_idx, k_idx, cand, nseg, seg, s);          \
  }
    MSA_FUSED_CASE(32, 64) MSA_FUSED_CASE(32, 128) MSA_FUSED_CASE(64, 64)
    MSA_FUSED_CASE(64, 128) MSA_FUSED_CASE(128, 64) MSA_FUSED_CASE(128, 128)
#undef MSA_FUSED_CASE
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)((p.total_q + 3) / 4), p.G);
  hipLaunchKernelGGL(index_topk_merge_kernel, grid, dim3(256), 0, s, cand, block_idx, p.cu_q,
                     p.cu_kv, p.num_seqs, p.B, p.top_k, nseg, seg, lst, p.total_q);
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace msa
