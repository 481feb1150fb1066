// Stable bucketing of kept-slot entries, shared by the backward passes.
//
// An entry e = row * K + slot of group g names kept slot `slot` of query row
// `row`.  A call buckets the entries [e_lo, e_hi) of every group (a range of
// whole rows: all of them, or one pass of a caller that runs its rows in
// passes); tiles and lists cover that range only.  Its bucket is the (sequence, block) pair the slot keeps, numbered
// b * nb_max + j within the group; padding slots and slots whose block holds
// no causal key of the row belong to no bucket.  Every bucket's list ends up
// in (row, slot) order, so sums taken in list order are deterministic:
//   bk_count     per tile of bucket_tile() consecutive entries of a group:
//                entries per bucket in an LDS histogram (integer atomics,
//                counting only)
//   bk_colscan   per bucket: exclusive offsets of the tiles, its total, its
//                number of work items of `per_item` entries, and its partial
//                slots (its items, when it has more than one)
//   bk_basescan  exclusive scan of the per-bucket totals / items / partials
//   bk_scatter   per tile, one wave walks its entries in order and writes
//                each to its bucket's list at tile offset + running count +
//                rank among equal buckets
#pragma once

#include "msa_common.hpp"

namespace msa {
namespace {

// Entries per counting / scatter tile: the scatter walks a tile with one
// wave, so small tiles run more of it in parallel, while the column scan
// walks the tiles of a bucket in order and every tile has a histogram of all
// of a group's buckets: 1024 entries, doubled up to 4096 while a group has
// more than 1024 tiles or more than 2^20 (tile, bucket) counts.
inline int64_t bucket_tile(int64_t nent_g, int64_t nbk_g) {
  int64_t t = 1024;
  while (t < 4096 && (nent_g > t * 1024 || (nent_g + t - 1) / t * nbk_g > (1 << 20))) t *= 2;
  return t;
}

// Bucket of entry e (= row * K + slot) of group g, or -1 when the slot is
// padding or its block holds no causal key of the row.  The bucket numbers
// blocks of every sequence: b * nb_max + j.  Also returns the row, the
// sequence's first key row and the row's position.
struct EntryInfo {
  int bucket;
  int64_t row, kv0, pos;
};
__device__ __forceinline__ EntryInfo entry_info(const int32_t *__restrict__ block_idx,
                                                const int64_t *__restrict__ cu_q,
                                                const int64_t *__restrict__ cu_kv, int num_seqs,
                                                int g, int64_t e, int K, int64_t total_q,
                                                int nb_max, int BS) {
  EntryInfo r;
  r.row = e / K;
  const int j = block_idx[(int64_t)g * total_q * K + e];
  const int b = find_seq(cu_q, num_seqs, r.row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  r.kv0 = sq.kv0;
  r.pos = sq.base + (r.row - sq.q0);
  const bool ok = j >= 0 && j < nb_max && r.pos >= 0 && (int64_t)j * BS <= r.pos;
  r.bucket = ok ? b * nb_max + j : -1;
  return r;
}

__global__ __launch_bounds__(256) void bk_count_kernel(
    const int32_t *__restrict__ block_idx, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int32_t *__restrict__ cnt, int32_t *__restrict__ amax,  // may be null
    int num_seqs, int K, int64_t total_q, int64_t e_lo, int64_t e_hi, int nb_max, int BS,
    int64_t ntiles, int64_t nbk_g, int64_t tile_len) {
  extern __shared__ int32_t hist[];  // [nbk_g]
  const int g = blockIdx.y;
  const int64_t tile = blockIdx.x;
  for (int64_t x = threadIdx.x; x < nbk_g; x += 256) hist[x] = 0;
  __syncthreads();
  const int64_t nent = total_q * K;  // entries of a group
  const int64_t e1 = min(e_hi, e_lo + (tile + 1) * tile_len);
  for (int64_t e = e_lo + tile * tile_len + threadIdx.x; e < e1; e += 256) {
    const EntryInfo ei = entry_info(block_idx, cu_q, cu_kv, num_seqs, g, e, K, total_q, nb_max, BS);
    if (ei.bucket >= 0) atomicAdd(&hist[ei.bucket], 1);
    else if (amax != nullptr) amax[(int64_t)g * nent + e] = -1;
  }
  __syncthreads();
  int32_t *dst = cnt + ((int64_t)g * ntiles + tile) * nbk_g;
  for (int64_t x = threadIdx.x; x < nbk_g; x += 256) dst[x] = hist[x];
}

// One thread per (group, bucket): tile counts -> exclusive tile offsets.
// amax (when not null) gets -1 for every entry that belongs to no bucket.
__global__ __launch_bounds__(256) void bk_colscan_kernel(int32_t *__restrict__ cnt,
                                                         int32_t *__restrict__ total,
                                                         int32_t *__restrict__ items,
                                                         int32_t *__restrict__ parts, int G,
                                                         int64_t ntiles, int64_t nbk_g,
                                                         int32_t per_item) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= (int64_t)G * nbk_g) return;
  const int64_t g = x / nbk_g, bk = x - g * nbk_g;
  int32_t run = 0;
  for (int64_t t = 0; t < ntiles; ++t) {
    int32_t *c = cnt + (g * ntiles + t) * nbk_g + bk;
    const int32_t v = *c;
    *c = run;
    run += v;
  }
  total[x] = run;
  const int32_t ni = (run + per_item - 1) / per_item;
  items[x] = ni;
  parts[x] = ni > 1 ? ni : 0;
}

// One work-group: exclusive scan of n bucket totals in place, base[n] = sum.
__global__ __launch_bounds__(1024) void bk_basescan_kernel(int32_t *__restrict__ base, int64_t n) {
  __shared__ int32_t part[1024];
  const int64_t per = (n + 1023) / 1024;
  const int64_t a = min(n, (int64_t)threadIdx.x * per), b = min(n, a + per);
  int32_t s = 0;
  for (int64_t i = a; i < b; ++i) s += base[i];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int32_t v = part[i];
      part[i] = run;
      run += v;
    }
    base[n] = run;
  }
  __syncthreads();
  int32_t run = part[threadIdx.x];
  for (int64_t i = a; i < b; ++i) {
    const int32_t v = base[i];
    base[i] = run;
    run += v;
  }
}

// One wave per (tile, group).  Chunks of 64 entries are placed in order: all
// lanes holding the same bucket are placed in one step, ranked by lane, after
// the tile's earlier entries of that bucket (a running count in LDS).
__global__ __launch_bounds__(64) void bk_scatter_kernel(
    const int32_t *__restrict__ block_idx, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, const int32_t *__restrict__ cnt,
    const int32_t *__restrict__ base, int32_t *__restrict__ lists, int num_seqs, int K,
    int64_t total_q, int64_t e_lo, int64_t e_hi, int nb_max, int BS, int64_t ntiles,
    int64_t nbk_g, int64_t tile_len) {
  extern __shared__ int32_t run[];  // [nbk_g] next list position of each bucket
  const int g = blockIdx.y;
  const int64_t tile = blockIdx.x;
  const int lane = threadIdx.x;
  // bucket start (global over groups) + this tile's offset in the bucket
  const int32_t *toff = cnt + ((int64_t)g * ntiles + tile) * nbk_g;
  const int32_t *gbase = base + (int64_t)g * nbk_g;
  for (int64_t x = lane; x < nbk_g; x += 64) run[x] = gbase[x] + toff[x];
  __syncthreads();
  const int64_t e1 = min(e_hi, e_lo + (tile + 1) * tile_len);
  for (int64_t c0 = e_lo + tile * tile_len; c0 < e1; c0 += 64) {
    const int64_t e = c0 + lane;
    int bk = -1;
    if (e < e1) bk = entry_info(block_idx, cu_q, cu_kv, num_seqs, g, e, K, total_q, nb_max, BS).bucket;
    bool active = bk >= 0;
    uint64_t act = ballot64(active);
    while (act != 0) {
      const int leader = (int)__builtin_ctzll(act);
      const int bl = __builtin_amdgcn_readlane(bk, leader);
      const uint64_t m = ballot64(active && bk == bl);
      const int32_t start = __builtin_amdgcn_readfirstlane(run[bl]);
      if (active && bk == bl) {
        MSA_DCHECK(start + (int32_t)mbcnt64(m) < gbase[bl + 1]);
        lists[start + mbcnt64(m)] = (int32_t)e;
        active = false;
      }
      if (lane == 0) run[bl] = start + __popcll(m);
      act = ballot64(active);
    }
  }
}

}  // namespace
}  // namespace msa
