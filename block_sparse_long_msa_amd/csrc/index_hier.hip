// Hierarchical (coarse-to-fine) block selection: an approximation of the
// Index Branch's selection that scores only a narrowed candidate set ("LongCat
// Sparse Attention" page, Abstract, strategy (3): a coarse-to-fine scoring
// scheme narrows each query's candidates to cut the indexing computation).
// Reading taken (the page gives no formula): chunks of S blocks carry a
// coarse key, the mean of their B*S index keys; a query at position p
// (current block J, current chunk cJ = J / S) scores its chunks c < cJ with
// <q_idx, coarse key>, keeps the C best (score descending, chunk ascending;
// all of them when there are at most C), and scores exactly (max-pooled
// dot products) the blocks of the kept chunks and the blocks of its current
// chunk below J; the k-1 best of those (score descending, block ascending)
// and J are kept.
//
// Kernels, in launch order:
//   hi_mean      coarse keys [num_seqs * nch, G, d_idx] fp32 of every full
//                chunk: four row quarters per column summed in order, then
//                added in order and scaled by 1 / (B * S) (a power of two)
//   hi_coarse    one wave per (group, row): the coarse scores of the chunks
//                below cJ (fp32, channel order), the C best by a bitwise
//                search over order-preserving keys with ballot counts (ties
//                to the lower chunk), listed ascending; slot C names the
//                current chunk when it holds blocks below J
//   bk_* (buckets.hpp)  the (row, slot) entries of every (sequence, chunk)
//   hi_fine      one work-group per work item (at most 256 entries of one
//                chunk's list): the chunk's blocks stream through a two-stage
//                LDS ring; the entries' gathered index queries are MFMA B
//                operands; each block's max-pooled score of every entry is
//                written where the block lies below the entry's J
//   hi_final     one wave per (group, row): the k-1 best fine candidates, in
//                ascending block order, and J
#include <algorithm>

#include "buckets.hpp"
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kHE = 256;  // entries per fine-scoring work item (4 waves x 64)

struct HiGeom {
  int S, C, K1;       // chunk blocks, kept chunks, slots per row (C + 1)
  int span;           // keys per chunk (B * S)
  int nch;            // chunks per sequence row of the coarse keys: ceil(NBmax / S)
};
HiGeom hi_geom(const Dims &p, int chunk_blocks, int keep_chunks) {
  HiGeom h;
  h.S = chunk_blocks;
  h.C = keep_chunks;
  h.K1 = keep_chunks + 1;
  h.span = p.B * chunk_blocks;
  h.nch = std::max(1, (p.nb_max + chunk_blocks - 1) / chunk_blocks);
  return h;
}

struct HiWs {
  float *kbar;       // [num_seqs * nch][G][d_idx]
  int32_t *sel;      // [G][total_q][K1] chunk of each slot (-1 none)
  float *fine;       // [G][total_q][K1][S] exact block scores of the slots' blocks
  int32_t *cnt, *base, *lists, *ibase, *pbase;   // stable bucketing (buckets.hpp)
  int64_t ntiles, nbk_g, nent_g, tile, max_items;
  size_t total_bytes;
};

size_t hal256(size_t x) { return (x + 255) & ~(size_t)255; }

HiWs hi_carve(const Dims &p, const HiGeom &h, void *base) {
  HiWs w;
  w.nent_g = p.total_q * (int64_t)h.K1;
  w.nbk_g = (int64_t)p.num_seqs * h.nch;
  w.tile = bucket_tile(w.nent_g, w.nbk_g);
  w.ntiles = std::max<int64_t>(1, (w.nent_g + w.tile - 1) / w.tile);
  size_t off = 0;
  char *c = static_cast<char *>(base);
  auto take = [&](size_t bytes) {
    char *r = c == nullptr ? nullptr : c + off;
    off += hal256(bytes);
    return r;
  };
  w.kbar = reinterpret_cast<float *>(take(sizeof(float) * (size_t)w.nbk_g * p.G * p.d_idx));
  w.sel = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)p.G * w.nent_g));
  w.fine = reinterpret_cast<float *>(take(sizeof(float) * (size_t)p.G * w.nent_g * h.S));
  w.cnt = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)p.G * w.ntiles * w.nbk_g));
  w.base = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  w.lists = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)p.G * w.nent_g));
  w.ibase = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  w.pbase = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  const int64_t nent = (int64_t)p.G * w.nent_g;
  w.max_items = nent / kHE + std::min<int64_t>((int64_t)p.G * w.nbk_g, nent) + 1;
  w.total_bytes = off;
  return w;
}

// Coarse keys: work-group (column block of 64, chunk, sequence); thread
// (quarter rq, column x) sums rows rq, rq + 4, ... of the chunk in order; the
// four quarter sums are added in order.  Only full chunks are written.
__global__ __launch_bounds__(256) void hi_mean_kernel(const uint16_t *__restrict__ k_idx,
                                                      float *__restrict__ kbar,
                                                      const int64_t *__restrict__ cu_kv, int G,
                                                      int DI, int span, int nch) {
  __shared__ float part[4][64];
  const int cols = G * DI;
  const int x = blockIdx.x * 64 + (threadIdx.x & 63), rq = threadIdx.x >> 6;
  const int c = blockIdx.y, b = blockIdx.z;
  const int64_t kv0 = cu_kv[b], lkv = cu_kv[b + 1] - kv0;
  if ((int64_t)(c + 1) * span > lkv) return;  // not a full chunk: never a coarse candidate
  float s = 0.f;
  if (x < cols) {
    const uint16_t *src = k_idx + (kv0 + (int64_t)c * span) * cols + x;
    for (int r = rq; r < span; r += 4) s += bf16_to_f32(src[(int64_t)r * cols]);
  }
  part[rq][threadIdx.x & 63] = s;
  __syncthreads();
  if (rq == 0 && x < cols) {
    const int l = threadIdx.x;
    const float tot = ((part[0][l] + part[1][l]) + part[2][l]) + part[3][l];
    kbar[((int64_t)b * nch + c) * cols + x] = tot * (1.f / (float)span);
  }
}

// Number of keys >= t (GE) or > t (!GE) over a wave's live slots (ballots).
template <int MAXS, bool GE>
__device__ __forceinline__ int hi_count(const uint32_t (&key)[MAXS], int live, uint32_t t) {
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < MAXS; ++u)
    if (u < live) cnt += __popcll(ballot64(GE ? key[u] >= t : key[u] > t));
  return cnt;
}

// Selection of the `want` largest order-preserving keys of a wave's live
// slots, ties to the first in (slot, lane) order: tau, the want-th largest
// key, by a bitwise search with ballot counts; every key above tau, then the
// first ties at tau until `want` are taken.  take[u] is set for the chosen.
template <int MAXS>
__device__ __forceinline__ void hi_select(const uint32_t (&key)[MAXS], int live, int want,
                                          bool (&take)[MAXS]) {
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = tau | (1u << bit);
    if (hi_count<MAXS, true>(key, live, t) >= want) tau = t;
  }
  const int c_gt = tau == 0xFFFFFFFFu ? 0 : hi_count<MAXS, false>(key, live, tau);
  int need = want - c_gt;  // ties at tau to take, first ones first
#pragma unroll
  for (int u = 0; u < MAXS; ++u) {
    const bool tie = u < live && key[u] == tau;
    const uint64_t m = ballot64(tie);
    take[u] = (u < live && key[u] > tau) || (tie && mbcnt64(m) < need);
    need -= min(need, __popcll(m));
  }
}

// One wave per (group, row), four rows of one group per work-group.
template <int DI, int MAXS>
__global__ __launch_bounds__(256) void hi_coarse_kernel(
    const uint16_t *__restrict__ q_idx, const float *__restrict__ kbar,
    int32_t *__restrict__ sel, int32_t *__restrict__ kept_out, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int num_seqs, int G, int BS, int S, int C, int K,
    int nch, int64_t total_q) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= total_q) return;
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  const int K1 = C + 1;
  int32_t *srow = sel + ((int64_t)g * total_q + row) * K1;
  int32_t *krow = kept_out == nullptr ? nullptr : kept_out + ((int64_t)g * total_q + row) * C;
  const int J = p < 0 ? -1 : (int)(p / BS);
  const int cJ = J < 0 ? 0 : J / S;
  // rows that keep 0..J without any score, and rows with no causal key, list nothing
  if (J <= K - 1) {
    for (int i = lane; i < K1; i += 64) srow[i] = -1;
    if (krow != nullptr)
      for (int i = lane; i < C; i += 64) krow[i] = i < cJ ? i : -1;
    return;
  }
  const int ncand = cJ;  // coarse candidates: chunks 0 .. cJ - 1
  const int live = (ncand + 63) >> 6;
  MSA_DCHECK(ncand <= 64 * MAXS && cJ <= nch);
  bool take[MAXS];
  if (ncand <= C) {
#pragma unroll
    for (int u = 0; u < MAXS; ++u) take[u] = u < live && lane + 64 * u < ncand;
  } else {
    // the query as fp32, read at a wave-uniform address
    float qf[DI];
    const uint16_t *qs = q_idx + (row * G + g) * (int64_t)DI;
#pragma unroll
    for (int i = 0; i < DI; i += 8) {
      const u32x4 w = ld16(qs + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[i + 2 * e] = bf16_lo(w[e]);
        qf[i + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
    uint32_t key[MAXS];
#pragma unroll
    for (int u = 0; u < MAXS; ++u) {
      key[u] = 0;
      const int c = lane + 64 * u;
      if (u < live && c < ncand) {
        const float *kb = kbar + (((int64_t)b * nch + c) * G + g) * DI;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < DI; i += 4) {
          const float4 kv = *reinterpret_cast<const float4 *>(kb + i);
          acc = fmaf(qf[i], kv.x, acc);
          acc = fmaf(qf[i + 1], kv.y, acc);
          acc = fmaf(qf[i + 2], kv.z, acc);
          acc = fmaf(qf[i + 3], kv.w, acc);
        }
        key[u] = ordered_key(acc);   // > 0 for every finite score
      }
    }
    hi_select<MAXS>(key, live, C, take);
  }
  // kept chunks ascending: (slot, lane) order is chunk order
  int at = 0;
#pragma unroll
  for (int u = 0; u < MAXS; ++u) {
    if (u >= live) break;
    const uint64_t m = ballot64(take[u]);
    MSA_DCHECK(!take[u] || at + (int)mbcnt64(m) < C);
    if (take[u]) {
      const int c = lane + 64 * u;
      srow[at + mbcnt64(m)] = c;
      if (krow != nullptr) krow[at + mbcnt64(m)] = c;
    }
    at += __popcll(m);
  }
  for (int i = at + lane; i < C; i += 64) {
    srow[i] = -1;
    if (krow != nullptr) krow[i] = -1;
  }
  if (lane == 0) srow[C] = cJ * S < J ? cJ : -1;  // the current chunk, if it has blocks below J
}

// Index-key block staging of the fine pass (same swizzle as the index kernels).
template <int DI, int BS>
struct HiTile {
  static constexpr int CPR = DI / 8;
  static constexpr int CHUNKS = BS * CPR;
  static constexpr int STAGE = CHUNKS * 16;
  static constexpr int RPB = 16 / CPR;
  __device__ static __forceinline__ int swz(int r, int q) { return r * CPR + (q ^ ((r / RPB) % CPR)); }
};

__device__ __forceinline__ void hi_dma16(const uint16_t *src, uint8_t *lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)lds, 16, 0, 0);
}

// One work-group (4 waves, 64 entries each) per work item.
template <int DI, int BS>
__global__ __launch_bounds__(256) void hi_fine_kernel(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    const int32_t *__restrict__ base, const int32_t *__restrict__ ibase,
    const int32_t *__restrict__ lists, float *__restrict__ fine, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int G, int K1, int S, int nch, int64_t total_q,
    int64_t nbuckets) {
  using T = HiTile<DI, BS>;
  constexpr int NW = 4;
  constexpr int KT = BS / 32, NK = DI / 16;
  constexpr int NLD = T::CHUNKS / 64, LPW = (NLD + NW - 1) / NW;
  static_assert(T::CHUNKS % 64 == 0, "whole 64-slot loads");
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[T::STAGE];
  __shared__ int32_t jmax_w[NW];
  const int32_t w = (int32_t)blockIdx.x;
  if (w >= ibase[nbuckets]) return;  // past the last item
  int64_t lo = 0, hi = nbuckets - 1;  // the bucket holding item w
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (ibase[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int64_t gb = lo;
  const int32_t it = w - ibase[gb];
  const int32_t n_b = base[gb + 1] - base[gb];
  const int32_t first = base[gb] + it * kHE, n = min(kHE, n_b - it * kHE);
  const int64_t nbk_g = nbuckets / G;
  const int g = (int)(gb / nbk_g);
  const int64_t bkt = gb - (int64_t)g * nbk_g;
  const int b = (int)(bkt / nch), c = (int)(bkt - (int64_t)b * nch);
  const int64_t kv0 = cu_kv[b], lkv = cu_kv[b + 1] - kv0;
  const int64_t q0 = cu_q[b], base_pos = lkv - (cu_q[b + 1] - q0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;

  // this lane's entry (after the block max, lane l of wave w holds entry 64w + l)
  const int x = wave * 64 + lane;
  const int32_t e = lists[first + min(x, n - 1)];
  const int64_t row = e / K1;
  const int slot = (int)(e - row * K1);
  const int J = (int)((base_pos + (row - q0)) / BS);   // >= c * S + 1 for every listed entry
  // the entry's row is a query of this bucket's sequence that lies past chunk c
  MSA_DCHECK(e >= 0 && row >= q0 && row < cu_q[b + 1] && slot < K1 && J >= c * S + 1);
  // blocks of the chunk below the largest J of the item
  int jm = x < n ? J : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) jm = max(jm, __shfl_xor(jm, off, 64));
  if (lane == 0) jmax_w[wave] = jm;
  __syncthreads();
  const int jmax = max(max(jmax_w[0], jmax_w[1]), max(jmax_w[2], jmax_w[3]));
  const int nblk = min(S, jmax - c * S);
  MSA_DCHECK((int64_t)(c * S + nblk) * BS <= lkv);

  // gathered index queries of the wave's two 32-column halves
  bf16x8 qb[2][NK];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int xe = min(wave * 64 + s * 32 + col, n - 1);
    const int64_t r = lists[first + xe] / K1;
    const uint16_t *src = q_idx + (r * G + g) * (int64_t)DI + 8 * half;
#pragma unroll
    for (int cc = 0; cc < NK; ++cc) qb[s][cc] = as_bf16x8(ld16(src + 16 * cc));
  }

  const int64_t kstride = (int64_t)G * DI;
  const uint16_t *kbase = k_idx + ((kv0 + (int64_t)c * S * BS) * G + g) * (int64_t)DI;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint16_t *kdma[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int Sl = min(64 * (wave_u + NW * i) + lane, T::CHUNKS - 1);
    const int r = Sl / T::CPR;
    kdma[i] = kbase + r * kstride + 8 * ((Sl % T::CPR) ^ ((r / T::RPB) % T::CPR));
  }
  const int64_t kblock = (int64_t)BS * kstride;
  auto dma = [&](int bi, uint8_t *dst) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int L = wave_u + NW * i;
      if (NLD % NW != 0 && L >= NLD) break;
      hi_dma16(kdma[i] + bi * kblock, dst + 1024 * L);
    }
  };
  float *frow = fine + (((int64_t)g * total_q + row) * K1 + slot) * S;
  auto block = [&](int bi, const uint8_t *cur) {
    float m0 = neg_inf(), m1 = neg_inf();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      u32x4 kf[NK];
      const int r = kt * 32 + col;
#pragma unroll
      for (int cc = 0; cc < NK; ++cc)
        kf[cc] = *reinterpret_cast<const u32x4 *>(cur + 16 * T::swz(r, 2 * cc + half));
      f32x16 a0 = {}, a1 = {};
#pragma unroll
      for (int cc = 0; cc < NK; ++cc) {
        a0 = mfma32x32x16(as_bf16x8(kf[cc]), qb[0][cc], a0);
        a1 = mfma32x32x16(as_bf16x8(kf[cc]), qb[1][cc], a1);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        m0 = fmaxf(m0, a0[i]);
        m1 = fmaxf(m1, a1[i]);
      }
    }
    const float m = halves_max_f(m0, m1);
    if (x < n && c * S + bi < J) frow[bi] = m;
  };
  // every block below jmax lies below some entry's position: all its keys exist
  dma(0, stage0);
  for (int bi = 0; bi < nblk; bi += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (bi + 1 < nblk) dma(bi + 1, stage1);
    block(bi, stage0);
    if (bi + 1 < nblk) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (bi + 2 < nblk) dma(bi + 2, stage0);
      block(bi + 1, stage1);
    }
  }
}

// One wave per (group, row): the k-1 best fine candidates and J.
template <int MAXS>
__global__ __launch_bounds__(256) void hi_final_kernel(
    const int32_t *__restrict__ sel, const float *__restrict__ fine,
    int32_t *__restrict__ block_idx, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int num_seqs, int BS, int S, int C, int K,
    int64_t total_q) {
  __shared__ int32_t pick[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= total_q) return;
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  int32_t *out = block_idx + ((int64_t)g * total_q + row) * K;
  if (p < 0) {
    for (int i = lane; i < K; i += 64) out[i] = -1;
    return;
  }
  const int J = (int)(p / BS);
  if (J <= K - 1) {
    for (int i = lane; i < K; i += 64) out[i] = i <= J ? i : -1;
    return;
  }
  if (K == 1) {
    if (lane == 0) out[0] = J;
    return;
  }
  const int K1 = C + 1;
  const int32_t *srow = sel + ((int64_t)g * total_q + row) * K1;
  const float *frow = fine + ((int64_t)g * total_q + row) * K1 * S;
  const int ncand = K1 * S;            // (slot, block) pairs, in ascending block order
  const int live = (ncand + 63) >> 6;
  uint32_t key[MAXS];
  int blk[MAXS];
#pragma unroll
  for (int u = 0; u < MAXS; ++u) {
    key[u] = 0;
    blk[u] = -1;
    const int i = lane + 64 * u;
    if (u < live && i < ncand) {
      const int slot = i / S, s = i - slot * S;
      const int c = srow[slot];
      const int j = c * S + s;
      if (c >= 0 && j < J) {
        key[u] = ordered_key(frow[i]);
        blk[u] = j;
      }
    }
  }
  bool take[MAXS];
  hi_select<MAXS>(key, live, K - 1, take);
  int at = 0;
#pragma unroll
  for (int u = 0; u < MAXS; ++u) {
    if (u >= live) break;
    const bool t = take[u] && blk[u] >= 0;
    const uint64_t m = ballot64(t);
    if (t) pick[wv][at + mbcnt64(m)] = blk[u];
    at += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // slot order is block order: the picks are ascending already
  for (int i = lane; i < K; i += 64) out[i] = i < at ? pick[wv][i] : (i == at ? J : -1);
}

template <int DI, int BS>
hipError_t launch_hier(const Dims &p, const HiGeom &h, const uint16_t *q_idx,
                       const uint16_t *k_idx, int32_t *block_idx, int32_t *kept_out,
                       void *workspace, hipStream_t s) {
  HiWs w = hi_carve(p, h, workspace);
  const int cols = p.G * DI;
  hipLaunchKernelGGL(hi_mean_kernel, dim3((unsigned)((cols + 63) / 64), h.nch, p.num_seqs),
                     dim3(256), 0, s, k_idx, w.kbar, p.cu_kv, p.G, DI, h.span, h.nch);
  profile_mark(s);
  const dim3 rows((unsigned)((p.total_q + 3) / 4), p.G);
  const int cmax = (h.nch + 63) / 64;  // coarse candidates per lane
  hipError_t e = hipErrorInvalidValue;
#define MSA_HC(M_)                                                                            \
  if (cmax <= M_) {                                                                           \
    hipLaunchKernelGGL((hi_coarse_kernel<DI, M_>), rows, dim3(256), 0, s, q_idx, w.kbar,    \
                       w.sel, kept_out, p.cu_q, p.cu_kv, p.num_seqs, p.G, p.B, h.S, h.C,     \
                       p.top_k, h.nch, p.total_q);                                            \
    e = hipSuccess;                                                                           \
  }
  MSA_HC(1) else MSA_HC(2) else MSA_HC(4) else MSA_HC(8) else MSA_HC(16)
#undef MSA_HC
  if (e != hipSuccess) return e;
  profile_mark(s);
  const size_t hist_bytes = sizeof(int32_t) * (size_t)w.nbk_g;
  hipLaunchKernelGGL(bk_count_kernel, dim3((unsigned)w.ntiles, p.G), dim3(256), hist_bytes, s,
                     w.sel, p.cu_q, p.cu_kv, w.cnt, nullptr, p.num_seqs, h.K1, p.total_q,
                     (int64_t)0, w.nent_g, h.nch, h.span, w.ntiles, w.nbk_g, w.tile);
  const int64_t ncol = (int64_t)p.G * w.nbk_g;
  hipLaunchKernelGGL(bk_colscan_kernel, dim3((unsigned)((ncol + 255) / 256)), dim3(256), 0, s,
                     w.cnt, w.base, w.ibase, w.pbase, p.G, w.ntiles, w.nbk_g, kHE);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.base, ncol);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.ibase, ncol);
  hipLaunchKernelGGL(bk_scatter_kernel, dim3((unsigned)w.ntiles, p.G), dim3(64), hist_bytes, s,
                     w.sel, p.cu_q, p.cu_kv, w.cnt, w.base, w.lists, p.num_seqs, h.K1,
                     p.total_q, (int64_t)0, w.nent_g, h.nch, h.span, w.ntiles, w.nbk_g, w.tile);
  profile_mark(s);
  hipLaunchKernelGGL((hi_fine_kernel<DI, BS>), dim3((unsigned)w.max_items), dim3(256), 0, s,
                     q_idx, k_idx, w.base, w.ibase, w.lists, w.fine, p.cu_q, p.cu_kv, p.G, h.K1,
                     h.S, h.nch, p.total_q, ncol);
  profile_mark(s);
  const int fmax = (h.K1 * h.S + 63) / 64;  // fine candidates per lane
  e = hipErrorInvalidValue;
#define MSA_HF(M_)                                                                              \
  if (fmax <= M_) {                                                                             \
    hipLaunchKernelGGL((hi_final_kernel<M_>), rows, dim3(256), 0, s, w.sel, w.fine, block_idx, \
                       p.cu_q, p.cu_kv, p.num_seqs, p.B, h.S, h.C, p.top_k, p.total_q);        \
    e = hipSuccess;                                                                             \
  }
  MSA_HF(2) else MSA_HF(4) else MSA_HF(8) else MSA_HF(16)
#undef MSA_HF
  if (e != hipSuccess) return e;
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace

MSA_DEBUG_COUNTER(index_hier)

bool hier_params_ok(const Dims &p, int chunk_blocks, int keep_chunks) {
  if (chunk_blocks < 1 || chunk_blocks > 64 || (chunk_blocks & (chunk_blocks - 1)) != 0)
    return false;
  if (keep_chunks < 1 || (int64_t)keep_chunks * chunk_blocks < p.top_k - 1) return false;
  const HiGeom h = hi_geom(p, chunk_blocks, keep_chunks);
  if ((int64_t)h.K1 * h.S > 64 * 16) return false;           // final pass slots
  if ((int64_t)h.nch > 64 * 16) return false;                // coarse pass slots
  if (p.total_q * (int64_t)h.K1 >= (int64_t)INT32_MAX) return false;
  if ((int64_t)p.num_seqs * h.nch * (int64_t)sizeof(int32_t) > 64 * 1024) return false;
  return true;
}

size_t hier_workspace_bytes(const Dims &p, int chunk_blocks, int keep_chunks) {
  if (p.total_q <= 0) return 0;
  return hi_carve(p, hi_geom(p, chunk_blocks, keep_chunks), nullptr).total_bytes;
}

hipError_t launch_index_topk_hier(const Dims &p, int chunk_blocks, int keep_chunks,
                                  const uint16_t *q_idx, const uint16_t *k_idx,
                                  int32_t *block_idx, int32_t *kept_chunks, void *workspace,
                                  hipStream_t s) {
  if (p.total_q <= 0) return hipSuccess;
  const HiGeom h = hi_geom(p, chunk_blocks, keep_chunks);
#define MSA_HI_CASE(DI_, BS_) \
  if (p.d_idx == DI_ && p.B == BS_)  \
    return launch_hier<DI_, BS_>(p, h, q_idx, k_idx, block_idx, kept_chunks, workspace, s);
  MSA_HI_CASE(32, 64) MSA_HI_CASE(32, 128) MSA_HI_CASE(64, 64) MSA_HI_CASE(64, 128)
  MSA_HI_CASE(128, 64) MSA_HI_CASE(128, 128)
#undef MSA_HI_CASE
  return hipErrorInvalidValue;
}

}  // namespace msa
