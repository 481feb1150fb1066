// Main Branch attention for prefill, KV-major ("MiniMax Sparse Attention"
// page: exact softmax attention restricted to the kept blocks, Summary,
// paragraph 2; the page's kernels order the loop KV-outer and balance skewed
// block popularity with pre-scheduled chunks and a two-phase combine without
// atomics, Summary paragraph 3 and Key points "Kernel design").
//
// Query-major gathering loads a 64 KiB K/V block for only H/G rows.  Here the
// loop is inverted: every kept (group, block) pair is one bucket holding the
// (query, slot) entries that kept it, and a work item stages ONE block in LDS
// and runs it against up to 256 gathered (query, head) rows with MFMA.  Each
// item writes an unnormalised partial result (sum of exp2(z - m) v in bf16,
// with the row's log2-domain max m and its sum l) for each of its entries,
// at the entry's own position: an item's results are one contiguous run, so
// the partial kernel's stores stream.  The scatter records that position per
// (query, slot of its kept-block list), and a merge kernel gathers and
// combines the slots of every (query, head) in slot order (deterministic, no
// atomics).
//
// Kernels, in launch order:
//   kv_clear        counts and cursors <- 0
//   kv_count        entries per bucket (integer atomics: only counting)
//   kv_scan_*       exclusive scan of the per-bucket work-item counts
//   kv_scatter      entry lists (t << 6 | slot) per bucket, item-major, and the
//                   position of each (query, slot) entry
//   kv_items        work-item descriptors (group, block, first entry, count, sequence)
//   kv_partial      persistent: one work-group per CU walks a contiguous range
//                   of work items (one bucket chunk of <= 256/hpg queries each),
//                   loading the next item while it computes the current one
//   kv_diag         the current (diagonal) block of every query, causal mask
//   kv_merge        per query: LSE-weighted merge of its slots -> out, lse
// Buckets never hold a query's current block: that block is shared by the
// whole 128-query block of positions, so kv_diag runs it densely.
#include <algorithm>
#include <atomic>

#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kRowsPerItem = 256;  // gathered (query, head) rows per work item
// Fewest query rows per pass when the workspace is too small for one pass.
constexpr int64_t kMinPassRows = 256;
// Long prefills run in passes whose gathered Q rows of one group take about
// this many bytes: such a pass's rows stay in the memory-side cache between
// the many reads of each row (one per kept block), which outweighs the
// passes' extra launches (measured at 128K; shorter problems run in one).
constexpr int64_t kPassQBytes = 32ll << 20;
constexpr int kWaves = 8;          // one 32-row tile per wave
constexpr int kThreads = 64 * kWaves;

// Buckets: one per (sequence, group, kept block), numbered
// (b * G + g) * nb_max + j.  (Splitting a bucket further by query chunk, so
// that a chunk's gathered Q rows stay in L2, was measured slower on the long
// prefill shapes: a chunk's bucket holds too few queries to fill work items,
// and every chunk re-reads the K/V block.)
constexpr int kScanTile = 4096;  // buckets per block of the item-count scan

struct KvWs {
  int32_t *counts, *cursor, *item_off, *entries, *scan_blk;
  int32_t *cbase;      // [nbk + 1] first entry of each bucket in entry order (scan of counts)
  int32_t *item_desc;  // per work item: g << 16 | j, 0, entry count, first KV row
  // Partials of the bucket entries in entry order (bucket after bucket, no
  // padding): entry c holds the H/G heads of its (row, kept block) pair.
  float2 *part_ml;     // [max_entries][H/G]     (m, l)
  uint16_t *part_o;    // [max_entries][H/G][d]  unnormalised O, bf16
  // Partials of the current block of every row of the pass (kv_diag).
  float2 *diag_ml;     // [rows][H]
  uint16_t *diag_o;    // [rows][H][d]
  int32_t *pmap;       // [G][rows][K]  entry index of each (row, kept block below J)
  uint16_t *trash_o;   // [64][d]  write target of lanes without a row (never read)
  float2 *trash_ml;    // [64]
  int64_t nbk, nscan, max_entries, max_items;
  size_t total_bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of one pass over at most `rows` consecutive query rows (the
// bucket arrays do not depend on it; entries, items and partials do).
KvWs carve(const Dims &p, void *base, int64_t rows) {
  KvWs w;
  w.nbk = (int64_t)p.num_seqs * p.G * p.nb_max;
  w.nscan = (w.nbk + kScanTile - 1) / kScanTile;
  w.max_entries = (int64_t)p.G * rows * p.top_k;
  const int qch = kRowsPerItem / (p.H / p.G);
  // every bucket adds at most one partly filled item
  w.max_items = w.max_entries / qch + std::min(w.nbk, w.max_entries) + 1;
  size_t off = 0;
  char *c = static_cast<char *>(base);
  auto take = [&](size_t bytes) {
    char *r = c == nullptr ? nullptr : c + off;
    off += align256(bytes);
    return r;
  };
  w.counts = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * w.nbk));
  w.cursor = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * w.nbk));
  w.item_off = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (w.nbk + 1)));
  w.cbase = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (w.nbk + 1)));
  w.scan_blk = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * 2 * (w.nscan + 1)));
  // item-major with qch slots per item (a bucket's last item is padded)
  w.entries = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * w.max_items * qch));
  w.item_desc = reinterpret_cast<int32_t *>(take(4 * sizeof(int32_t) * w.max_items));
  const int64_t hpg = p.H / p.G;
  w.part_ml = reinterpret_cast<float2 *>(take(sizeof(float2) * w.max_entries * hpg));
  w.part_o = reinterpret_cast<uint16_t *>(take(sizeof(uint16_t) * w.max_entries * hpg * p.d));
  w.diag_ml = reinterpret_cast<float2 *>(take(sizeof(float2) * rows * p.H));
  w.diag_o = reinterpret_cast<uint16_t *>(take(sizeof(uint16_t) * rows * p.H * p.d));
  w.pmap = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * p.G * rows * p.top_k));
  w.trash_o = reinterpret_cast<uint16_t *>(take(sizeof(uint16_t) * 64 * p.d));
  w.trash_ml = reinterpret_cast<float2 *>(take(sizeof(float2) * 64));
  w.total_bytes = off;
  return w;
}

// Row position helpers shared by the schedule kernels.
struct RowInfo {
  int b;
  int64_t p;  // absolute position of the query (negative: no causal key)
};
__device__ __forceinline__ RowInfo row_info(const int64_t *cu_q, const int64_t *cu_kv,
                                            int num_seqs, int64_t row) {
  RowInfo r;
  r.b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, r.b);
  r.p = sq.base + (row - sq.q0);
  return r;
}

__global__ __launch_bounds__(256) void kv_clear_kernel(int32_t *a, int32_t *b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    a[i] = 0;
    b[i] = 0;
  }
}

// Count and scatter work on tiles of kEntTile consecutive (row, slot) entries
// of one group.  Entries are kept blocks strictly below the query's current
// block (all their keys are causal).  Buckets of the tile's first sequence
// are counted in an LDS histogram over the block index first, so a tile
// issues one global atomic per touched bucket instead of one per entry; rows
// of another sequence (tiles that straddle a boundary) go straight to global
// atomics.  The order of entries inside a bucket is not
// fixed, but every entry's result is computed independently of its
// neighbours, so outputs do not depend on it.
constexpr int kEntPerThread = 32;
constexpr int kEntTile = 256 * kEntPerThread;

struct EntryRef {
  int64_t bkt;   // bucket, or -1 if the entry is not a partial-attention entry
  int bin;       // LDS bin (block index) if the entry is in the tile's first sequence, else -1
};

// Geometry shared by the count and scatter kernels.  kmagic = ceil(2^32 / K)
// splits a tile-local entry offset x < 2^16 into (row, slot) exactly:
// x / K = (x * kmagic) >> 32 (the rounding error of kmagic is below K, and
// x * K < 2^32).  Block sizes are powers of two: J = p >> lg_bs.
struct EntGeom {
  int G, K, lg_bs, nb_max, num_seqs;
  uint32_t kmagic_lo, kmagic_hi;  // ceil(2^32 / K) as two words (it is 2^32 for K = 1)
  int64_t total_q;                // row stride of block_idx's groups
  int64_t row_lo, nrows;          // the pass's query rows [row_lo, row_lo + nrows)
};

// Entries of one tile: the pass-local entry index el = (row - row_lo) * K +
// slot runs over [el0, el0 + kEntTile); thread entry i of the tile is
// el0 + tid + 256 i.
struct TileStart {
  int64_t el0, row0;  // the tile's first entry and its row
  int off0;           // its slot
  int b0;             // sequence of row0
  int64_t bbase;      // first bucket of (b0, g)
  SeqGeom s0;
};
struct EntPos {
  int64_t row;
  int slot;
};
__device__ __forceinline__ EntPos entry_pos(const TileStart &t, const EntGeom &cg, int local) {
  const uint32_t x = (uint32_t)(t.off0 + local);  // < K + kEntTile < 2^16
  const uint64_t magic = ((uint64_t)cg.kmagic_hi << 32) | cg.kmagic_lo;
  const uint32_t q = (uint32_t)(((uint64_t)x * magic) >> 32);
  return EntPos{t.row0 + q, (int)(x - q * (uint32_t)cg.K)};
}

__device__ __forceinline__ EntryRef entry_ref(const int32_t *__restrict__ block_idx, int64_t e,
                                              const EntPos &ep, int g, const EntGeom &cg,
                                              const TileStart &t, const int64_t *cu_q,
                                              const int64_t *cu_kv) {
  EntryRef r{-1, -1};
  const int j = block_idx[e];
  if (j < 0) return r;
  int b = t.b0;
  SeqGeom sq = t.s0;
  if (ep.row < t.s0.q0 || ep.row >= t.s0.q0 + t.s0.lq) {
    b = find_seq(cu_q, cg.num_seqs, ep.row);
    sq = seq_geom(cu_q, cu_kv, b);
  }
  const int64_t p = sq.base + (ep.row - sq.q0);
  if (p < 0 || (int64_t)j >= (p >> cg.lg_bs)) return r;
  MSA_DCHECK(j < cg.nb_max && b >= 0 && b < cg.num_seqs);
  r.bkt = ((int64_t)b * cg.G + g) * cg.nb_max + j;
  r.bin = b == t.b0 ? j : -1;
  return r;
}

__device__ __forceinline__ TileStart tile_start(int g, const EntGeom &cg, const int64_t *cu_q,
                                                const int64_t *cu_kv) {
  TileStart t;
  t.el0 = (int64_t)blockIdx.x * kEntTile;
  const int64_t lrow = t.el0 / cg.K;  // once per work-group
  t.off0 = (int)(t.el0 - lrow * cg.K);
  t.row0 = cg.row_lo + lrow;
  t.b0 = find_seq(cu_q, cg.num_seqs, t.row0);
  t.s0 = seq_geom(cu_q, cu_kv, t.b0);
  t.bbase = ((int64_t)t.b0 * cg.G + g) * cg.nb_max;
  return t;
}

__global__ __launch_bounds__(256) void kv_count_kernel(const int32_t *__restrict__ block_idx,
                                                       int32_t *__restrict__ counts,
                                                       const int64_t *__restrict__ cu_q,
                                                       const int64_t *__restrict__ cu_kv,
                                                       EntGeom cg) {
  extern __shared__ int32_t hist[];  // nb_max bins
  const int g = blockIdx.y;
  const int64_t per_g = cg.nrows * cg.K;
  const TileStart ts = tile_start(g, cg, cu_q, cu_kv);
  const int n = (int)min<int64_t>(kEntTile, per_g - ts.el0);
  if (n <= 0) return;
  const int32_t *bi = block_idx + ((int64_t)g * cg.total_q + cg.row_lo) * cg.K + ts.el0;
  for (int i = threadIdx.x; i < cg.nb_max; i += 256) hist[i] = 0;
  __syncthreads();
  for (int local = threadIdx.x; local < n; local += 256) {
    const EntryRef r = entry_ref(bi, local, entry_pos(ts, cg, local), g, cg, ts, cu_q, cu_kv);
    if (r.bin >= 0) atomicAdd(&hist[r.bin], 1);
    else if (r.bkt >= 0) atomicAdd(&counts[r.bkt], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < cg.nb_max; i += 256)
    if (hist[i] != 0) atomicAdd(&counts[ts.bbase + i], hist[i]);
}

// Entries are laid out item-major: the bucket's entry of rank `pos` goes to
// item_off[bucket] * qch + pos, so work item t owns entries [t*qch, t*qch + qch).
// An entry is stored as row << 6 | slot.  Its partial result goes to entry
// index cbase[bucket] + pos (the same order without the padding of the last
// items), which pmap[g][row][slot] records for the merge.
__global__ __launch_bounds__(256) void kv_scatter_kernel(const int32_t *__restrict__ block_idx,
                                                         int32_t *__restrict__ cursor,
                                                         const int32_t *__restrict__ item_off,
                                                         const int32_t *__restrict__ cbase,
                                                         int32_t *__restrict__ entries,
                                                         int32_t *__restrict__ pmap,
                                                         const int64_t *__restrict__ cu_q,
                                                         const int64_t *__restrict__ cu_kv,
                                                         EntGeom cg, int qch) {
  // nb_max bins: local counts, then the tile's base per bin; then the
  // tile's base per bin in entry-index order
  extern __shared__ int32_t hist[];
  int32_t *hist2 = hist + cg.nb_max;
  const int g = blockIdx.y;
  const int64_t per_g = cg.nrows * cg.K;
  const TileStart ts = tile_start(g, cg, cu_q, cu_kv);
  const int n = (int)min<int64_t>(kEntTile, per_g - ts.el0);
  if (n <= 0) return;
  const int32_t *bi = block_idx + ((int64_t)g * cg.total_q + cg.row_lo) * cg.K + ts.el0;
  for (int i = threadIdx.x; i < cg.nb_max; i += 256) hist[i] = 0;
  __syncthreads();
  int rank[kEntPerThread];
#pragma unroll
  for (int i = 0; i < kEntPerThread; ++i) {
    const int local = threadIdx.x + 256 * i;
    rank[i] = -1;
    if (local < n) {
      const EntPos ep = entry_pos(ts, cg, local);
      const EntryRef r = entry_ref(bi, local, ep, g, cg, ts, cu_q, cu_kv);
      if (r.bin >= 0) {
        rank[i] = atomicAdd(&hist[r.bin], 1);
      } else if (r.bkt >= 0) {
        const int pos = atomicAdd(&cursor[r.bkt], 1);
        MSA_DCHECK(pos < (item_off[r.bkt + 1] - item_off[r.bkt]) * qch);
        entries[item_off[r.bkt] * qch + pos] = (int32_t)((ep.row << 6) | ep.slot);
        pmap[((int64_t)g * cg.nrows + (ep.row - cg.row_lo)) * cg.K + ep.slot] = cbase[r.bkt] + pos;
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < cg.nb_max; i += 256) {
    const int c = hist[i];
    const int pb = c != 0 ? atomicAdd(&cursor[ts.bbase + i], c) : 0;
    hist[i] = c != 0 ? item_off[ts.bbase + i] * qch + pb : 0;
    hist2[i] = c != 0 ? cbase[ts.bbase + i] + pb : 0;
    // the tile's run of the bucket ends inside the bucket's items
    MSA_DCHECK(c == 0 || hist[i] + c <= item_off[ts.bbase + i + 1] * qch);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kEntPerThread; ++i) {
    if (rank[i] < 0) continue;
    const int local = threadIdx.x + 256 * i;
    const EntPos ep = entry_pos(ts, cg, local);
    const int j = bi[local];
    entries[hist[j] + rank[i]] = (int32_t)((ep.row << 6) | ep.slot);
    pmap[((int64_t)g * cg.nrows + (ep.row - cg.row_lo)) * cg.K + ep.slot] = hist2[j] + rank[i];
  }
}

// Exclusive scans of the per-bucket work-item counts ceil(count / qch) into
// item_off and of the entry counts into cbase (item_off[nbk], cbase[nbk] =
// totals), in three passes: per block of kScanTile buckets a local scan and
// the block's totals; a single work-group scan of the block totals; then
// each block adds its offsets.  scan_blk holds the item totals, then (at
// nscan + 1) the entry totals.
__device__ __forceinline__ int32_t block_excl_scan256(int32_t v, int32_t *sh, int32_t *total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
    const int32_t add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int32_t incl = sh[tid];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(256) void kv_scan_local_kernel(const int32_t *__restrict__ counts,
                                                            int32_t *__restrict__ item_off,
                                                            int32_t *__restrict__ cbase,
                                                            int32_t *__restrict__ scan_blk,
                                                            int64_t nbk, int64_t nscan, int qch) {
  __shared__ int32_t sh[256];
  constexpr int PER = kScanTile / 256;
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * PER;
  int32_t v[PER], c[PER];
  int32_t sum_v = 0, sum_c = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t bk = base + i;
    c[i] = bk < nbk ? counts[bk] : 0;
    v[i] = (c[i] + qch - 1) / qch;
    sum_v += v[i];
    sum_c += c[i];
  }
  int32_t tot_v, tot_c;
  int32_t run_v = block_excl_scan256(sum_v, sh, &tot_v);
  int32_t run_c = block_excl_scan256(sum_c, sh, &tot_c);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t bk = base + i;
    if (bk < nbk) {
      item_off[bk] = run_v;
      cbase[bk] = run_c;
    }
    run_v += v[i];
    run_c += c[i];
  }
  if (threadIdx.x == 0) {
    scan_blk[blockIdx.x] = tot_v;
    scan_blk[nscan + 1 + blockIdx.x] = tot_c;
  }
}

__global__ __launch_bounds__(256) void kv_scan_top_kernel(int32_t *__restrict__ scan_blk,
                                                          int64_t nscan) {
  __shared__ int32_t sh[256];
  for (int part = 0; part < 2; ++part) {  // item totals, then entry totals
    int32_t *a = scan_blk + part * (nscan + 1);
    int32_t carry = 0;
    for (int64_t b0 = 0; b0 < nscan; b0 += 256) {
      const int64_t i = b0 + threadIdx.x;
      const int32_t v = i < nscan ? a[i] : 0;
      int32_t total;
      const int32_t ex = block_excl_scan256(v, sh, &total);
      if (i < nscan) a[i] = carry + ex;
      carry += total;
    }
    if (threadIdx.x == 0) a[nscan] = carry;
  }
}

__global__ __launch_bounds__(256) void kv_scan_add_kernel(int32_t *__restrict__ item_off,
                                                          int32_t *__restrict__ cbase,
                                                          const int32_t *__restrict__ scan_blk,
                                                          int64_t nbk, int64_t nscan) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nbk) {
    item_off[i] += scan_blk[i / kScanTile];
    cbase[i] += scan_blk[nscan + 1 + i / kScanTile];
  }
  if (i == 0) {
    item_off[nbk] = scan_blk[nscan];
    cbase[nbk] = scan_blk[2 * nscan + 1];
  }
}

// One wave per bucket (four buckets per work-group): the lanes write the
// descriptors of the bucket's work items (g << 16 | block, entry index of the
// item's first entry, entry count, packed row of the block's first key), so a
// work item starts after one 16-byte load and no divisions, and fill the
// unused entry slots of the bucket's last item with the pass's first row /
// slot 0 (a valid row to load; the partial kernel never stores for those
// lanes).
__global__ __launch_bounds__(256) void kv_items_kernel(const int32_t *__restrict__ counts,
                                                       const int32_t *__restrict__ item_off,
                                                       const int32_t *__restrict__ cbase,
                                                       int32_t *__restrict__ entries,
                                                       int32_t *__restrict__ item_desc,
                                                       const int64_t *__restrict__ cu_kv,
                                                       int64_t nbk, int G, int nb_max, int BS,
                                                       int qch, int32_t pad_entry) {
  const int lane = threadIdx.x & 63;
  const int64_t bkt = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (bkt >= nbk) return;
  const int cnt = counts[bkt];
  if (cnt == 0) return;
  const int first = item_off[bkt];
  const uint32_t c0 = (uint32_t)cbase[bkt];
  const int64_t t = bkt / nb_max;  // scalar, once per bucket
  const uint32_t j = (uint32_t)(bkt - t * nb_max);
  const int64_t b = t / G;
  const uint32_t g = (uint32_t)(t - b * G);
  const uint32_t kvrow = (uint32_t)(cu_kv[b] + (int64_t)j * BS);
  const int nitems = (cnt + qch - 1) / qch;
  for (int i = lane; i < nitems; i += 64) {
    u32x4 d = {g << 16 | j, c0 + (uint32_t)(i * qch), (uint32_t)min(qch, cnt - i * qch), kvrow};
    st16(item_desc + 4 * (int64_t)(first + i), d);
  }
  for (int i = cnt + lane; i < nitems * qch; i += 64) entries[(int64_t)first * qch + i] = pad_entry;
}

// LDS tile of one K/V block, both row-major [key][d] without padding.  The
// 16-byte chunks of each row are XOR-swizzled (chunk c of row r sits at
// c ^ swz(r)) so that the MFMA operand reads spread over all LDS banks:
//   K: swz = r mod (D/8); the S^T operand read takes 32 consecutive rows at
//      one chunk.
//   V: swz = 2 (r mod 4) + 8 ((r / 4) mod 2) (D = 128; D = 64 drops the
//      second term); the transposed read takes 4 consecutive rows x 32 bytes
//      per 16 lanes.
// The tile is filled by direct HBM -> LDS loads (16 bytes per lane, lane L
// of a load writing LDS bytes [16L, 16L + 16) of the load's base), so the
// swizzle is applied by choosing which global chunk each lane fetches.
template <int D, int BS>
struct KvTile {
  uint16_t k[BS * D];
  uint16_t v[BS * D];
};
template <int D>
__device__ __forceinline__ int k_swz(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? 2 * (r & 3) + 8 * ((r >> 2) & 1) : 2 * (r & 3);
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// Issues the direct loads of block rows [key0, key0 + BS) of group g (packed
// row kvrow0 + key) into tile t.  With CLAMP, keys at or past nvalid read
// key nvalid - 1 instead (their scores are masked; V then holds finite
// values that are multiplied by zero).  Completion is waited for by the
// caller (vmcnt, then a barrier before other waves read the tile).
template <int D, int BS, bool CLAMP>
__device__ __forceinline__ void dma_kv(KvTile<D, BS> &t, const uint16_t *__restrict__ k,
                                       const uint16_t *__restrict__ v, int64_t kvrow0,
                                       int nvalid, int G, int g) {
  constexpr int CPR = D / 8;              // chunks per row
  constexpr int NCH = BS * CPR;           // chunks per tensor
  constexpr int PER_WAVE = NCH / kWaves;  // chunks per wave, a multiple of 64
  static_assert(PER_WAVE % 64 == 0, "whole 64-lane loads per wave");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rs = (int64_t)G * D;
  const uint16_t *kb = k + (kvrow0 * G + g) * (int64_t)D;
  const uint16_t *vb = v + (kvrow0 * G + g) * (int64_t)D;
#pragma unroll
  for (int i = 0; i < PER_WAVE / 64; ++i) {
    const int p0 = wave * PER_WAVE + i * 64;  // first chunk of this load (wave-uniform)
    const int p = p0 + lane;
    const int row = p / CPR, cp = p % CPR;
    const int key = CLAMP ? min(row, nvalid - 1) : row;
    __builtin_amdgcn_global_load_lds(kb + key * rs + 8 * (cp ^ k_swz<D>(row)),
                                     (lds_void *)(t.k + 8 * p0), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + key * rs + 8 * (cp ^ v_swz<D>(row)),
                                     (lds_void *)(t.v + 8 * p0), 16, 0, 0);
  }
}

// Reads back one element of this wave's own part of tile t and pins it: the
// compiler then waits for this wave's loads into t right here (and no later
// than here), so a barrier placed after this call publishes the tile.
template <int D, int BS>
__device__ __forceinline__ void dma_settle(const KvTile<D, BS> &t) {
  constexpr int PER_WAVE = BS * D / 8 / kWaves;
  const int wave = threadIdx.x >> 6;
  uint32_t x = *reinterpret_cast<const volatile uint16_t *>(t.k + 8 * (wave * PER_WAVE + PER_WAVE - 1)) +
               *reinterpret_cast<const volatile uint16_t *>(t.v + 8 * (wave * PER_WAVE + PER_WAVE - 1));
  asm volatile("" : "+v"(x));
}

// All V^T fragments of one dv tile: for 16-key step ks, the transposed reads
// at key rows 16ks (+ 4 half + l/4, folded into `addr`) and 16ks + 8, as
// immediate offsets from `addr` (an LDS byte address).  One asm block issues
// every read and waits for them before it ends.  The tile being read was
// published by a barrier before this point, while the direct loads in flight
// target the other tile: written as builtins, these reads would make the
// compiler wait for those loads, as it cannot tell the two tiles apart.
// The outputs are early-clobber (=&v): the first read writes its result
// before the later reads have used `addr`, so no output may share the
// address register.
#define MSA_TR(i) "ds_read_b64_tr_b16 %" #i ", %[a] offset:%[o" #i "]\n"
template <int D, int BS>
__device__ __forceinline__ void vt_tile_read(u32x4 (&aw)[BS / 16], uint32_t addr) {
  constexpr int R = 2 * D;  // bytes per V row
  u32x2 x[BS / 8];
  if constexpr (BS == 128) {
    asm volatile(MSA_TR(0) MSA_TR(1) MSA_TR(2) MSA_TR(3) MSA_TR(4) MSA_TR(5) MSA_TR(6) MSA_TR(7)
                 MSA_TR(8) MSA_TR(9) MSA_TR(10) MSA_TR(11) MSA_TR(12) MSA_TR(13) MSA_TR(14)
                 MSA_TR(15) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
                   "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]),
                   "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15])
                 : [a] "v"(addr), [o0] "n"(0 * R), [o1] "n"(8 * R), [o2] "n"(16 * R),
                   [o3] "n"(24 * R), [o4] "n"(32 * R), [o5] "n"(40 * R), [o6] "n"(48 * R),
                   [o7] "n"(56 * R), [o8] "n"(64 * R), [o9] "n"(72 * R), [o10] "n"(80 * R),
                   [o11] "n"(88 * R), [o12] "n"(96 * R), [o13] "n"(104 * R), [o14] "n"(112 * R),
                   [o15] "n"(120 * R));
  } else {
    static_assert(BS == 64, "block size 64 or 128");
    asm volatile(MSA_TR(0) MSA_TR(1) MSA_TR(2) MSA_TR(3) MSA_TR(4) MSA_TR(5) MSA_TR(6) MSA_TR(7)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
                   "=&v"(x[6]), "=&v"(x[7])
                 : [a] "v"(addr), [o0] "n"(0 * R), [o1] "n"(8 * R), [o2] "n"(16 * R),
                   [o3] "n"(24 * R), [o4] "n"(32 * R), [o5] "n"(40 * R), [o6] "n"(48 * R),
                   [o7] "n"(56 * R));
  }
#pragma unroll
  for (int ks = 0; ks < BS / 16; ++ks)
    aw[ks] = u32x4{x[2 * ks][0], x[2 * ks][1], x[2 * ks + 1][0], x[2 * ks + 1][1]};
}
#undef MSA_TR

// K fragments of MFMA step c for the four 32-key tiles of a 128-key block
// (rows kt*32 + col, kt = 0..3): the K swizzle depends on col mod 16 only, so
// the four reads share one LDS byte address `addr` and differ by immediate
// offsets; one asm block issues them and waits before it ends (same reason,
// and the same early-clobber outputs, as vt_tile_read).
template <int D>
__device__ __forceinline__ void k_step_read4(u32x4 (&kf)[4], uint32_t addr) {
  constexpr int T = 32 * 2 * D;  // bytes per 32-key tile
  asm volatile(
      "ds_read_b128 %0, %[a] offset:%[o0]\n"
      "ds_read_b128 %1, %[a] offset:%[o1]\n"
      "ds_read_b128 %2, %[a] offset:%[o2]\n"
      "ds_read_b128 %3, %[a] offset:%[o3]\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3])
      : [a] "v"(addr), [o0] "n"(0), [o1] "n"(T), [o2] "n"(2 * T), [o3] "n"(3 * T));
}

// Q^T operands of one lane's row (B operand of S^T = K . Q^T): 16 values of
// d per MFMA step, lanes 0-31 and 32-63 taking the two halves of each step.
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qb)[D / 16], const uint16_t *qrow, bool valid) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qb[c] = valid ? as_bf16x8(ld16(qrow + 16 * c + 8 * half)) : zero_bf16x8();
}

// Partial O rows are stored with d permuted to the MFMA result layout, so a
// lane writes its 16 values of a 32-wide dv tile as 32 contiguous bytes:
// stored position 32*dt + 16*half + 4*i + e holds dv = 32*dt + 8*i + 4*half + e.
__device__ __forceinline__ int partial_dv(int pos) {
  const int dt = pos >> 5, half = (pos >> 4) & 1, i = (pos >> 2) & 3, e = pos & 3;
  return 32 * dt + 8 * i + 4 * half + e;
}

// One wave, 32 rows (MFMA columns) against the staged block:
//   S^T (keys x rows) = K . Q^T, softmax per row (log2 domain), O^T = V^T . P^T.
// The lane's row has Q operands `qb` and position `pos` (keys s0 + key > pos
// are masked when MASK).  Writes the unnormalised O = sum_s exp2(z_s - m) v_s
// (bf16, permuted d) and (m, l) to `o_dst` / `ml_dst`, where z_s are the
// log2-domain logits, m their max and l = sum_s exp2(z_s - m).  Every lane
// stores (lanes without a row of their own point at scratch rows): stores
// outside divergent branches keep the memory counters' waits exact.
// WIDE keeps more operands in flight (independent accumulators for the four
// key tiles of S^T, a whole dv tile of V^T read ahead of its MFMAs) for
// kernels with a 256-register budget; the narrow form fits 128 registers.
template <int D, int BS, bool MASK, bool WIDE>
__device__ __forceinline__ void attend_rows(const KvTile<D, BS> &t, const bf16x8 (&qb)[D / 16],
                                            int64_t s0, int64_t pos, float scale_log2,
                                            uint16_t *o_dst, float2 *ml_dst) {
  constexpr int NC = D / 16;     // MFMA steps over d
  constexpr int KT = BS / 32;    // 32-key tiles
  constexpr int DT = D / 32;     // 32-wide dv tiles
  const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
  // S^T: the four key tiles accumulate independently, so consecutive MFMAs
  // never wait on each other.
  f32x16 s[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) s[kt] = f32x16{};
  // K fragment of key tile kt, MFMA step c: row kt*32 + col, chunk 2c + half
  auto k_op = [&](int kt, int c) {
    const int r = kt * 32 + col;
    return *reinterpret_cast<const u32x4 *>(t.k + r * D + 8 * ((2 * c + half) ^ k_swz<D>(r)));
  };
  if constexpr (WIDE && KT == 4) {
    // the four key tiles accumulate independently; the fragments of step c
    // are read in one block while the MFMAs of step c - 1 run
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 kf[4];
      k_step_read4<D>(kf, (uint32_t)(uintptr_t)(t.k + col * D + 8 * ((2 * c + half) ^ k_swz<D>(col))));
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) s[kt] = mfma32x32x16(as_bf16x8(kf[kt]), qb[c], s[kt]);
    }
  } else if constexpr (WIDE) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) s[kt] = mfma32x32x16(as_bf16x8(k_op(kt, c)), qb[c], s[kt]);
    }
  } else {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int c = 0; c < NC; ++c) s[kt] = mfma32x32x16(as_bf16x8(k_op(kt, c)), qb[c], s[kt]);
      __builtin_amdgcn_sched_barrier(0);  // one key tile's operands live at a time
    }
  }
  // max over the raw logits (the scale is positive), masked keys at -inf
  float mraw = neg_inf();
  // causal limit inside the block: keys with local index > lim are masked
  const int lim = MASK ? (int)min<int64_t>(max<int64_t>(pos - s0, -1), BS) : BS;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (MASK && kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) > lim) s[kt][r] = neg_inf();
      mraw = fmaxf(mraw, s[kt][r]);
    }
  }
  mraw = xor32_max_f(mraw);
  const float m = mraw * scale_log2;  // max of the log2-domain logits
  const float msafe = mraw == neg_inf() ? 0.f : m;
  // P in bf16, one 16-key MFMA step at a time: step ks takes registers
  // 8*(ks&1) .. +7 of S^T tile ks/2, i.e. keys 16ks + 4*half + {0..3} and
  // 16ks + 8 + 4*half + {0..3}; V^T is read below with the same key order.
  u32x4 pk[BS / 16];
  float l = 0.f;
#pragma unroll
  for (int ks = 0; ks < BS / 16; ++ks) {
    const int r0 = 8 * (ks & 1);
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][r0 + i], scale_log2, -msafe));
      l += e[i];
    }
    pk[ks] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                   pack_bf16x2(e[6], e[7])};
  }
  l = xor32_sum_f(l);
  // V^T fragments of dv tile dt, read transposed from the row-major V tile:
  // within each 16-lane group, lane l points at key row r0 + l/4 and dv
  // 4(l%4) .. +3 of its group's 16 dv; lane i then receives V[r0 .. r0+3][dv
  // of lane i].  Step ks takes rows r0 = 16ks + 4half and 16ks + 8 + 4half,
  // the key order of pk.  Along a lane's reads only r0 changes by multiples
  // of 8 and the V swizzle of its rows stays 2 (l/4) + 8 half, so all of a
  // tile's reads share one address and differ by immediate offsets.
  const int lq = lane & 15;
  auto vt_base = [&](int dt) {
    const int dv = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lq & 3);
    const int r = 4 * half + (lq >> 2);
    return (uint32_t)(uintptr_t)(t.v + r * D + 8 * ((dv >> 3) ^ v_swz<D>(r)) + (dv & 7));
  };
  // o[4i + e] is dv = 32dt + 8i + 4half + e: stored at 32dt + 16half + 4i + e
  auto store_o = [&](int dt, const f32x16 &o) {
    uint16_t *dst = o_dst + 32 * dt + 16 * half;
    u32x4 w0 = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                pack_bf16x2(o[6], o[7])};
    u32x4 w1 = {pack_bf16x2(o[8], o[9]), pack_bf16x2(o[10], o[11]), pack_bf16x2(o[12], o[13]),
                pack_bf16x2(o[14], o[15])};
    st16(dst, w0);
    st16(dst + 8, w1);
  };
  if constexpr (WIDE) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x4 aw[BS / 16];
      vt_tile_read<D, BS>(aw, vt_base(dt));
      f32x16 o = {};
#pragma unroll
      for (int ks = 0; ks < BS / 16; ++ks) o = mfma32x32x16(as_bf16x8(aw[ks]), as_bf16x8(pk[ks]), o);
      store_o(dt, o);
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x4 aw[BS / 16];
      vt_tile_read<D, BS>(aw, vt_base(dt));
      f32x16 o = {};
#pragma unroll
      for (int ks = 0; ks < BS / 16; ++ks) o = mfma32x32x16(as_bf16x8(aw[ks]), as_bf16x8(pk[ks]), o);
      store_o(dt, o);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // both halves hold the same (m, l) and store it to the same place
  *ml_dst = l > 0.f ? float2{m, l} : float2{neg_inf(), 0.f};
}

// Hands the tile that this wave has been loading over to the other waves:
// waits until this wave's direct loads into it have landed and meets them at
// a barrier.  The vector memory counter completes in issue order, and the
// last NAFTER vector memory operations issued before this point (the current
// item's partial-result stores) come after those loads, so vmcnt <= NAFTER
// is enough; the stores keep draining.  There is no memory fence: the LDS
// tile is all that is exchanged, and a fence would wait for the stores.  The
// LDS reads of the current tile waited for themselves (asm blocks).
template <int NAFTER>
__device__ __forceinline__ void tile_handover() {
  static_assert(NAFTER >= 0 && NAFTER < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((NAFTER & 15) | (7 << 4) | (15 << 8) | ((NAFTER >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Decoded work-item descriptor (see kv_items_kernel).
struct ItemDesc {
  int g, n;
  int64_t kvrow;  // packed K/V row of the block's first key
  int64_t c0;     // entry index of the item's first entry (its partials start there)
};

// A zero the compiler cannot see through: addresses built from it are
// per-lane, so loads through them stay vector loads (counted by vmcnt, in
// order with the other vector memory traffic) instead of scalar loads.
__device__ __forceinline__ int opaque_lane_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Pins a value in place: instructions that read it cannot be scheduled above
// this point (the empty asm "rewrites" it), and the value must be ready here.
__device__ __forceinline__ void pin(u32x4 &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(int32_t &x) { asm volatile("" : "+v"(x)); }

// Persistent partial attention.  Work-groups are dealt to the XCDs
// round-robin (work-group w runs on XCD w % 8); the item order is described
// at the top of the kernel.  Each work-group double-buffers the K/V tile in
// LDS: while it
// computes item t from one tile, the K/V block of item t+1 streams straight
// into the other tile, its Q rows into registers, and the descriptor and
// entries of item t+2 too; one barrier per item hands the tiles over.  Every
// lane owns one (query, head) row of each item.
//
// The loop is unrolled by two so that the two sets of Q registers and item
// metadata trade roles instead of being copied (a copy of a register that a
// load is still filling would make the compute wait for that load), and it
// has no data-dependent branch around a memory access: lanes past an item's
// rows load a valid row and store to scratch rows, and a work-group with an
// odd item count runs its last item twice (same values to the same places).
template <int D, int BS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void kv_partial_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ item_off,
    const int32_t *__restrict__ entries, const int32_t *__restrict__ item_desc,
    uint16_t *__restrict__ part_o, float2 *__restrict__ part_ml, uint16_t *__restrict__ trash_o,
    float2 *__restrict__ trash_ml, int H, int G, [[maybe_unused]] int K, int nseg, int nb_max,
    int qch, float scale_log2, [[maybe_unused]] int64_t row_lo, [[maybe_unused]] int64_t row_hi,
    [[maybe_unused]] int64_t total_kv, [[maybe_unused]] int64_t max_entries) {
  static_assert(kRowsPerItem == 32 * kWaves, "one 32-row tile per wave");
  // two separate objects, so the compiler can tell the tile being loaded
  // from the tile being read
  __shared__ __attribute__((aligned(16))) KvTile<D, BS> tile_a;
  __shared__ __attribute__((aligned(16))) KvTile<D, BS> tile_b;
  // Item order.  Items come in segments, one per (sequence, group) pair (its
  // buckets, block by block).  Every XCD takes its eighth of segment 0, then
  // its eighth of segment 1, and so on, and the XCD's work-groups stride
  // through that eighth: at any time the whole GPU gathers Q rows of the
  // same group (a working set that stays in the Infinity Cache between the
  // many reads of each row), and consecutive items of an XCD still share
  // buckets (the K/V block stays in its L2).
  int xcd = 0, parts = 1, nw = gridDim.x, w = blockIdx.x;
  if (gridDim.x % 8 == 0) {
    xcd = blockIdx.x % 8;
    parts = 8;
    nw = gridDim.x / 8;
    w = blockIdx.x / 8;
  }
  auto part_of = [&](int sg, int &plo, int &phi) {
    const int a = item_off[(int64_t)sg * nb_max], b = item_off[(int64_t)(sg + 1) * nb_max];
    plo = a + (int)((int64_t)(b - a) * xcd / parts);
    phi = a + (int)((int64_t)(b - a) * (xcd + 1) / parts);
  };
  int total = 0;  // items of this work-group
  for (int sg = 0; sg < nseg; ++sg) {
    int plo, phi;
    part_of(sg, plo, phi);
    if (plo + w < phi) total += (phi - plo - w + nw - 1) / nw;
  }
  if (total == 0) return;
  // Cursor over this work-group's items; once they run out it repeats the
  // last one (a work-group with an odd count runs its last item twice,
  // writing the same values to the same places).
  int cur_sg = 0, cur_it = 0, cur_end = 0, cur_last = 0;
  auto next_item = [&]() {
    while (cur_it >= cur_end && cur_sg < nseg) {
      int plo, phi;
      part_of(cur_sg, plo, phi);
      ++cur_sg;
      cur_it = plo + w;
      cur_end = phi;
    }
    if (cur_it < cur_end) {
      cur_last = cur_it;
      cur_it += nw;
    }
    return cur_last;
  };
  const int hpg = H / G;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, col = lane & 31;
  const int r = wave * 32 + col;   // this lane's row of every item
  const int qi = r / hpg;          // query of the item
  const int hh = r - qi * hpg;     // head inside the group
  const int qs = min(qi, qch - 1); // entry slot read by this lane
  const int32_t *desc_base = item_desc + opaque_lane_zero();
  auto meta_at = [&](int it, u32x4 &wd, int32_t &e) {
    wd = ld16(desc_base + 4 * (int64_t)it);
    e = entries[(int64_t)it * qch + qs];
  };
  auto decode = [&](const u32x4 &w) {
    ItemDesc d;
    d.g = (int)(__builtin_amdgcn_readfirstlane(w[0]) >> 16);
    d.n = (int)__builtin_amdgcn_readfirstlane(w[2]);
    d.kvrow = (int64_t)__builtin_amdgcn_readfirstlane(w[3]);
    d.c0 = (int64_t)__builtin_amdgcn_readfirstlane(w[1]);
    return d;
  };
  auto q_of = [&](bf16x8 (&qb)[D / 16], const ItemDesc &d, int32_t e) {
    MSA_DCHECK(e >= 0 && (e >> 6) >= row_lo && (e >> 6) < row_hi && (e & 63) < K && d.g >= 0 &&
               d.g < G);
    MSA_DCHECK(d.kvrow >= 0 && d.kvrow + BS <= total_kv);
    const int half = lane >> 5;
    const uint16_t *qrow = q + ((int64_t)(e >> 6) * H + d.g * hpg + hh) * (int64_t)D + 8 * half;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qb[c] = as_bf16x8(ld16(qrow + 16 * c));
  };
  // One item: prefetch the next item's data (metadata wn / en: Q rows to
  // registers, K/V block straight into tile tn) and the metadata of the one
  // after (into wc / ec, free once the current item's store addresses are
  // formed), then compute the current item from tile tc.
  auto run_item = [&](int it_after_next, bf16x8 (&qc)[D / 16], bf16x8 (&qn)[D / 16], u32x4 &wc,
                      int32_t &ec, u32x4 &wn, int32_t &en, KvTile<D, BS> &tc,
                      KvTile<D, BS> &tn) {
    // the next item's metadata is read from here on, not earlier (where it
    // would make the previous compute wait for its load)
    pin(wn);
    pin(en);
    const ItemDesc dc = decode(wc);
    const bool own = qi < dc.n;
    // the partial goes to the entry's index in entry order, so an item's
    // stores fill one contiguous range
    MSA_DCHECK(!own || dc.c0 + qi < max_entries);
    const int64_t ps = (dc.c0 + qi) * hpg + hh;
    uint16_t *od = own ? part_o + ps * D : trash_o + lane * D;
    float2 *md = own ? part_ml + ps : trash_ml + lane;
    const ItemDesc dn = decode(wn);
    q_of(qn, dn, en);
    dma_kv<D, BS, false>(tn, k, v, dn.kvrow, BS, G, dn.g);
    meta_at(it_after_next, wc, ec);
    // keep the loads above ahead of the compute (the scheduler would
    // otherwise sink them next to their first use, after it)
    __builtin_amdgcn_sched_barrier(0);
    attend_rows<D, BS, false, true>(tc, qc, 0, 0, scale_log2, od, md);
    // the item's stores: two 16-byte stores per 32-wide dv tile, then (m, l)
    tile_handover<2 * (D / 32) + 1>();
  };

  u32x4 wa, wb;
  int32_t ea, eb;
  meta_at(next_item(), wa, ea);
  meta_at(next_item(), wb, eb);
  bf16x8 qa[D / 16], qb[D / 16];
  {
    const ItemDesc d = decode(wa);
    q_of(qa, d, ea);
    dma_kv<D, BS, false>(tile_a, k, v, d.kvrow, BS, G, d.g);
  }
  dma_settle<D, BS>(tile_a);
  __syncthreads();
  for (int done = 0; done < total; done += 2) {
    run_item(next_item(), qa, qb, wa, ea, wb, eb, tile_a, tile_b);
    run_item(next_item(), qb, qa, wb, eb, wa, ea, tile_b, tile_a);
  }
}

// The current block of each 128-query block of positions, with the causal
// mask; every row's partial goes to its row of the diagonal buffer (the merge
// uses it when the row's list holds that block).
template <int D, int BS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void kv_diag_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ diag_o, float2 *__restrict__ diag_ml,
    uint16_t *__restrict__ trash_o, float2 *__restrict__ trash_ml,
    const int64_t *__restrict__ cu_q, const int64_t *__restrict__ cu_kv, int H, int G,
    int nb_max, float scale_log2, int64_t row_lo, int64_t row_hi) {
  __shared__ __attribute__((aligned(16))) KvTile<D, BS> tile;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  // the sequence's local queries in this pass
  const int64_t ilo = max<int64_t>(0, row_lo - sq.q0), ihi = min<int64_t>(sq.lq, row_hi - sq.q0);
  if (ihi <= ilo) return;
  // blockIdx.x counts the blocks that hold those queries, from the block of
  // the first one at a non-negative position
  const int J = (int)(max<int64_t>(sq.base + ilo, 0) / BS) + blockIdx.x;
  if (J >= nb_max) return;
  // local queries of the pass whose position lies in block J
  const int64_t i0 = max<int64_t>(ilo, (int64_t)J * BS - sq.base);
  const int64_t i1 = min<int64_t>(ihi, (int64_t)(J + 1) * BS - sq.base);
  if (i1 <= i0) return;
  const int64_t s0 = (int64_t)J * BS;
  const int hpg = H / G;
  const int nrows = (int)(i1 - i0) * hpg;
  const int wave = threadIdx.x >> 6, col = threadIdx.x & 31;
  // row tile rt -> (valid, query row, position, head)
  struct RowT {
    bool valid;
    int64_t row, pos;
    int h;
  };
  auto row_of = [&](int rt) {
    RowT x;
    const int r = rt * 32 + col;
    x.valid = r < nrows;
    const int qi = x.valid ? r / hpg : 0;
    const int hh = x.valid ? r - qi * hpg : 0;
    x.row = sq.q0 + i0 + qi;
    x.pos = sq.base + i0 + qi;
    x.h = g * hpg + hh;
    return x;
  };
  dma_kv<D, BS, true>(tile, k, v, sq.kv0 + s0, (int)min<int64_t>(BS, sq.lkv - s0), G, g);
  dma_settle<D, BS>(tile);
  __syncthreads();
  for (int rt = wave; rt * 32 < nrows; rt += kWaves) {
    const RowT cur = row_of(rt);
    bf16x8 qa[D / 16];
    load_q<D>(qa, q + (cur.row * H + cur.h) * (int64_t)D, cur.valid);
    const int64_t ps = (cur.row - row_lo) * H + cur.h;
    const int lane = threadIdx.x & 63;
    attend_rows<D, BS, true, false>(tile, qa, s0, cur.pos, scale_log2,
                             cur.valid ? diag_o + ps * D : trash_o + lane * D,
                             cur.valid ? diag_ml + ps : trash_ml + lane);
  }
}

// Per query row: merge the slots whose block is causal (0 <= j <= J).
// Phase 0 finds, per (group, slot), where that slot's partial lies: the
// entry position pmap recorded for a block below J, the row of the diagonal
// buffer for the last slot listing J, or nothing (-1).  Phase 1 spreads the
// (slot, head) pairs over the work-group: each loads its slot's (m, l) (m =
// -inf for unused slots) into LDS; then one thread per head forms M = max m,
// the weights w = exp2(m - M) (0 for unused slots) and 1 / sum(w l).  Phase 2
// gathers the bf16 partials (the H/G heads of an entry are one contiguous
// run), each thread owning 8 consecutive output values of one head, with the
// slot loop unrolled so several 16-byte loads are in flight.  Unused slots
// read the row's diagonal partial (valid memory) and are never multiplied:
// the select below drops them.
// With block_mass set, the kernel also writes the Main Branch distribution
// over each group's kept blocks (the target of the indexer's KL objective,
// "MiniMax Sparse Attention" page, Summary, paragraph 2): head h puts
// w l / L of its softmax on slot sl, and the group's heads are averaged.
template <int D>
__global__ __launch_bounds__(256) void kv_merge_kernel(
    const int32_t *__restrict__ block_idx, const uint16_t *__restrict__ part_o,
    const float2 *__restrict__ part_ml, const uint16_t *__restrict__ diag_o,
    const float2 *__restrict__ diag_ml, const int32_t *__restrict__ pmap,
    uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ block_mass,
    const int64_t *__restrict__ cu_q, const int64_t *__restrict__ cu_kv, int num_seqs, int H,
    int G, int K, int BS, int64_t total_q, int64_t row_lo, [[maybe_unused]] int64_t nslots) {
  extern __shared__ float wsh[];  // [K][H] m, then weights; [K][H] l; [H] 1/sum; [K][G] sources
  float *lsh = wsh + K * H;
  float *winv = lsh + K * H;
  int32_t *src_sh = reinterpret_cast<int32_t *>(winv + H);
  constexpr int kDiag = -2, kNone = -1;
  const int64_t nrows = gridDim.x;    // rows of the pass
  const int64_t lrow = blockIdx.x;    // row of the pass (its partials)
  const int64_t row = row_lo + lrow;  // query row
  constexpr int OPH = D / 8;  // octets per head (of stored, d-permuted partial positions)
  const RowInfo ri = row_info(cu_q, cu_kv, num_seqs, row);
  const int64_t J = ri.p < 0 ? -1 : ri.p / BS;
  const int hpg = H / G;
  for (int t = threadIdx.x; t < G * K; t += 256) {
    const int g = t / K, sl = t - g * K;
    const int32_t *br = block_idx + ((int64_t)g * total_q + row) * K;
    const int j = br[sl];
    int src = kNone;
    if (j >= 0 && j < J) {
      src = pmap[((int64_t)g * nrows + lrow) * K + sl];
      MSA_DCHECK(src >= 0 && src < nslots);
    } else if (J >= 0 && j == J) {  // the last slot listing J takes the diagonal partial
      src = kDiag;
      for (int s2 = sl + 1; s2 < K; ++s2)
        if (br[s2] == J) src = kNone;
    }
    src_sh[sl * G + g] = src;
  }
  __syncthreads();
  // (slot, head) pairs in batches of four per thread: the (m, l) of a batch
  // are all requested before any is used
  for (int t0 = threadIdx.x; t0 < K * H; t0 += 4 * 256) {
    int src[4];
    float2 mlr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = min(t0 + 256 * u, K * H - 1);
      const int sl = t / H, h = t - sl * H;
      src[u] = src_sh[sl * G + h / hpg];
      const float2 *p = src[u] >= 0 ? part_ml + (int64_t)src[u] * hpg + (h - (h / hpg) * hpg)
                                    : diag_ml + lrow * H + h;
      mlr[u] = *p;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + 256 * u;
      if (t >= K * H) break;
      const float2 ml = src[u] != kNone ? mlr[u] : float2{neg_inf(), 0.f};
      wsh[t] = ml.y > 0.f ? ml.x : neg_inf();
      lsh[t] = ml.y;
    }
  }
  __syncthreads();
  for (int h = threadIdx.x; h < H; h += 256) {
    float M = neg_inf();
    for (int sl = 0; sl < K; ++sl) M = fmaxf(M, wsh[sl * H + h]);
    float L = 0.f;
    for (int sl = 0; sl < K; ++sl) {
      const float ms = wsh[sl * H + h];
      const float w = (M == neg_inf() || ms == neg_inf()) ? 0.f : exp2f(ms - M);
      wsh[sl * H + h] = w;
      L += w * lsh[sl * H + h];
    }
    winv[h] = L > 0.f ? 1.f / L : 0.f;
    if (lse != nullptr) lse[row * H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : neg_inf();
  }
  __syncthreads();
  if (block_mass != nullptr) {
    // unused slots have w = 0 and l = 0; a row without causal keys has 1/L = 0
    for (int t = threadIdx.x; t < G * K; t += 256) {
      const int g = t / K, sl = t - g * K;
      float pm = 0.f;
      for (int h = g * hpg; h < (g + 1) * hpg; ++h) pm += wsh[sl * H + h] * lsh[sl * H + h] * winv[h];
      block_mass[((int64_t)g * total_q + row) * K + sl] = pm / (float)hpg;
    }
  }
  for (int oc = threadIdx.x; oc < H * OPH; oc += 256) {
    const int h = oc / OPH, g = h / hpg;
    const int o8 = oc - h * OPH;
    // element offset of the head's octet inside an entry, and the diagonal row's
    const int64_t in_entry = (int64_t)(h - g * hpg) * D + 8 * o8;
    const uint16_t *dsrc = diag_o + (lrow * H + h) * (int64_t)D + 8 * o8;
    auto slot_src = [&](int sl) {
      const int e = src_sh[sl * G + g];
      return e >= 0 ? part_o + (int64_t)e * hpg * D + in_entry : dsrc;
    };
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 4 <= K; s += 4) {
      u32x4 x[4];
      float w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w[u] = wsh[(s + u) * H + h];
        x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(slot_src(s + u)));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += w[u] > 0.f ? w[u] * bf16_lo(x[u][i]) : 0.f;
          acc[2 * i + 1] += w[u] > 0.f ? w[u] * bf16_hi(x[u][i]) : 0.f;
        }
      }
    }
    for (; s < K; ++s) {
      const float w = wsh[s * H + h];
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(slot_src(s)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w > 0.f ? w * bf16_lo(x[i]) : 0.f;
        acc[2 * i + 1] += w > 0.f ? w * bf16_hi(x[i]) : 0.f;
      }
    }
    const float inv = winv[h];
    // the 8 stored positions 8*o8 .. +7 are two runs of 4 consecutive dv
    const int dv0 = partial_dv(8 * o8), dv1 = partial_dv(8 * o8 + 4);
    uint16_t *orow = out + row * (int64_t)H * D + (int64_t)h * D;
    u32x2 r0 = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    u32x2 r1 = {pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
    *reinterpret_cast<u32x2 *>(orow + dv0) = r0;
    *reinterpret_cast<u32x2 *>(orow + dv1) = r1;
  }
}

// Work-groups of the persistent partial kernel: one per compute unit (its
// two LDS tiles take most of a CU's 160 KiB), never more than the items.
int persistent_grid(int64_t max_items) {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return (int)std::max<int64_t>(1, std::min<int64_t>(n, max_items));
}

// LDS of the merge: (m, l) of every (slot, head), 1 / sum per head, and the
// source of every (slot, group).
size_t merge_lds_bytes(const Dims &p) {
  return sizeof(float) * (2 * (size_t)p.top_k * p.H + p.H) +
         sizeof(int32_t) * (size_t)p.top_k * p.G;
}

// One pass of the KV-major path over query rows [row_lo, row_hi): bucket
// the pass's kept-slot entries, run the partial, diagonal and merge kernels.
// Each row's result depends on its own entries only, so splitting the rows
// into passes changes no output bit.
template <int D, int BS>
void launch_pass(const Dims &p, const KvWs &w, int64_t row_lo, int64_t row_hi,
                 const uint16_t *q, const uint16_t *k, const uint16_t *v,
                 const int32_t *block_idx, uint16_t *out, float *lse, float *block_mass,
                 hipStream_t s) {
  const int64_t nrows = row_hi - row_lo;
  const int hpg = p.H / p.G;
  const int qch = kRowsPerItem / hpg;
  const float sl2 = p.scale * kLog2e;
  hipLaunchKernelGGL(kv_clear_kernel, dim3((unsigned)((w.nbk + 255) / 256)), dim3(256), 0, s,
                     w.counts, w.cursor, w.nbk);
  profile_mark(s);
  const uint64_t kmagic = ((1ull << 32) + (uint64_t)p.top_k - 1) / (uint64_t)p.top_k;
  const EntGeom cg{p.G, p.top_k, 31 - __builtin_clz(p.B), p.nb_max, p.num_seqs,
                   (uint32_t)kmagic, (uint32_t)(kmagic >> 32), p.total_q, row_lo, nrows};
  const int64_t per_g = nrows * p.top_k;
  const dim3 tiles((unsigned)((per_g + kEntTile - 1) / kEntTile), p.G);
  const size_t hist_bytes = sizeof(int32_t) * p.nb_max;
  hipLaunchKernelGGL(kv_count_kernel, tiles, dim3(256), hist_bytes, s, block_idx, w.counts,
                     p.cu_q, p.cu_kv, cg);
  profile_mark(s);
  hipLaunchKernelGGL(kv_scan_local_kernel, dim3((unsigned)w.nscan), dim3(256), 0, s, w.counts,
                     w.item_off, w.cbase, w.scan_blk, w.nbk, w.nscan, qch);
  hipLaunchKernelGGL(kv_scan_top_kernel, dim3(1), dim3(256), 0, s, w.scan_blk, w.nscan);
  hipLaunchKernelGGL(kv_scan_add_kernel, dim3((unsigned)((w.nbk + 255) / 256)), dim3(256), 0, s,
                     w.item_off, w.cbase, w.scan_blk, w.nbk, w.nscan);
  profile_mark(s);
  hipLaunchKernelGGL(kv_scatter_kernel, tiles, dim3(256), 2 * hist_bytes, s, block_idx, w.cursor,
                     w.item_off, w.cbase, w.entries, w.pmap, p.cu_q, p.cu_kv, cg, qch);
  profile_mark(s);
  hipLaunchKernelGGL(kv_items_kernel, dim3((unsigned)((w.nbk + 3) / 4)), dim3(256), 0, s,
                     w.counts, w.item_off, w.cbase, w.entries, w.item_desc, p.cu_kv, w.nbk, p.G,
                     p.nb_max, p.B, qch, (int32_t)(row_lo << 6));
  profile_mark(s);
  hipLaunchKernelGGL((kv_partial_kernel<D, BS>), dim3((unsigned)persistent_grid(w.max_items)),
                     dim3(kThreads), 0, s, q, k, v, w.item_off, w.entries, w.item_desc, w.part_o,
                     w.part_ml, w.trash_o, w.trash_ml, p.H, p.G, p.top_k, p.num_seqs * p.G,
                     p.nb_max, qch, sl2, row_lo, row_hi, p.total_kv, w.max_entries);
  profile_mark(s);
  // the blocks holding a sequence's queries of the pass: at most
  // ceil(min(max_q_len, nrows) / B) + 1
  const int64_t span = std::min<int64_t>(p.max_q_len, nrows);
  const int ndiag = (int)std::min<int64_t>((span + p.B - 1) / p.B + 1, p.nb_max);
  hipLaunchKernelGGL((kv_diag_kernel<D, BS>), dim3(ndiag, p.G, p.num_seqs), dim3(kThreads), 0, s,
                     q, k, v, w.diag_o, w.diag_ml, w.trash_o, w.trash_ml, p.cu_q, p.cu_kv,
                     p.H, p.G, p.nb_max, sl2, row_lo, row_hi);
  profile_mark(s);
  hipLaunchKernelGGL((kv_merge_kernel<D>), dim3((unsigned)nrows), dim3(256), merge_lds_bytes(p), s,
                     block_idx, w.part_o, w.part_ml, w.diag_o, w.diag_ml, w.pmap, out, lse,
                     block_mass, p.cu_q, p.cu_kv, p.num_seqs, p.H, p.G, p.top_k, p.B, p.total_q,
                     row_lo, w.max_entries);
  profile_mark(s);
}

template <int D, int BS>
hipError_t launch_all(const Dims &p, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const int32_t *block_idx, uint16_t *out, float *lse, float *block_mass,
                      void *workspace, int64_t rows_per_pass, hipStream_t s) {
  const KvWs w = carve(p, workspace, rows_per_pass);
  for (int64_t r0 = 0; r0 < p.total_q; r0 += rows_per_pass) {
    launch_pass<D, BS>(p, w, r0, std::min(p.total_q, r0 + rows_per_pass), q, k, v, block_idx,
                       out, lse, block_mass, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

MSA_DEBUG_COUNTER(attn_kvmajor)

bool kvmajor_fits(const Dims &p) {
  if (p.total_q >= (int64_t)1 << 25) return false;  // entries pack the query row above 6 slot bits
  // the merge keeps (m, l) of every (slot, head) of a row in LDS
  if (merge_lds_bytes(p) > 64 * 1024) return false;
  const KvWs w = carve(p, nullptr, p.total_q);
  return w.max_items * (kRowsPerItem / (p.H / p.G)) < (int64_t)INT32_MAX;
}

size_t kvmajor_workspace_bytes(const Dims &p, int64_t rows_per_pass) {
  return carve(p, nullptr, std::max<int64_t>(1, std::min(rows_per_pass, p.total_q))).total_bytes;
}

size_t kvmajor_workspace_min_bytes(const Dims &p) { return kvmajor_workspace_bytes(p, kMinPassRows); }

int64_t kvmajor_preferred_rows(const Dims &p) {
  const int64_t row_bytes = (int64_t)(p.H / p.G) * p.d * 2;
  return std::max<int64_t>(kMinPassRows, kPassQBytes / row_bytes);
}

int64_t kvmajor_rows_per_pass(const Dims &p, size_t workspace_bytes) {
  if (kvmajor_workspace_bytes(p, p.total_q) <= workspace_bytes) return p.total_q;
  if (kvmajor_workspace_bytes(p, kMinPassRows) > workspace_bytes) return 0;
  int64_t lo = std::min<int64_t>(kMinPassRows, p.total_q), hi = p.total_q;  // fits, does not
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (kvmajor_workspace_bytes(p, mid) <= workspace_bytes) lo = mid; else hi = mid;
  }
  return lo;
}

hipError_t launch_attn_kvmajor_bf16(const Dims &p, const uint16_t *q, const uint16_t *k,
                                    const uint16_t *v, const int32_t *block_idx, uint16_t *out,
                                    float *lse, float *block_mass, void *workspace,
                                    int64_t rows_per_pass, hipStream_t s) {
  if (p.total_q <= 0) return hipSuccess;
  if (rows_per_pass <= 0) return hipErrorInvalidValue;
#define MSA_KV_CASE(D_, BS_) \
  if (p.d == D_ && p.B == BS_)  \
    return launch_all<D_, BS_>(p, q, k, v, block_idx, out, lse, block_mass, workspace, \
                               rows_per_pass, s);
  MSA_KV_CASE(64, 64) MSA_KV_CASE(64, 128) MSA_KV_CASE(128, 64) MSA_KV_CASE(128, 128)
#undef MSA_KV_CASE
  return hipErrorInvalidValue;
}

}  // namespace msa
