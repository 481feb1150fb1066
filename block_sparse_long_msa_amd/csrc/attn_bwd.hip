// Backward of the Main Branch ("MiniMax Sparse Attention" page, Summary,
// paragraph 2: exact softmax attention restricted to the keys of the kept
// blocks).  For row t and head h of group g, with z_s = scale <q, k_s> over
// the kept causal keys, P = softmax(z) (rebuilt from the forward's LSE) and
// an upstream gradient dO of the output:
//   D        = <dO, O>                       (= sum_s P_s <dO, v_s>)
//   dS_s     = P_s (<dO, v_s> - D)
//   dv_s    += P_s dO          dk_s += scale dS_s q          dq += scale dS_s k_s
//
// KV-major, like the forward's KV-major schedule (the page's kernels loop
// KV-outer): every (sequence, group, kept block) bucket lists the (row, slot)
// entries that kept the block, the current block included (its causal mask
// is applied per row), in (row, slot) order (buckets.hpp).  A work item is
// up to kSteps steps of one bucket's list; a step is 64 (query, head) rows.
// The item keeps its block's K and V in LDS for all its steps and
// accumulates dK, dV of the block in registers; every step writes the rows'
// dQ contribution of this block into the row's slot (bf16), which a merge
// then sums in slot order.  No floating-point atomics: every sum has a fixed
// order.
//
// Kernels, in launch order:
//   ab_dsum      D = rowsum(dO * O) per (row, head)
//   bk_*         bucket lists and work items (buckets.hpp)
//   ab_zero_unkept  dk, dv <- 0 on the keys of blocks no slot keeps
//   ab_item      per work item: S = Q K^T, dP = dO V^T, P, dS with MFMA; dV^T
//                += dO^T P, dK^T += Q^T dS, dQ^T = K^T dS^T
//   ab_reduce    per bucket of several items: dk, dv = the items' partial
//                sums added in item order
//   ab_dq        per (row, head): dq = scale * sum of its slots' dQ, in slot order
#include <algorithm>

#include "buckets.hpp"
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kD = 128;           // head dimension
constexpr int kBS = 128;          // block size
constexpr int kRows = 64;         // (query, head) rows per step
constexpr int kSteps = 64;        // steps per work item
constexpr int kItemThreads = 512;  // 8 waves: 4 key groups x 2 halves

struct AbWs {
  int32_t *cnt, *base, *lists, *ibase, *pbase;
  float *dsum;        // [total_q][H] rowsum(dO * O)
  uint16_t *dq_part;  // [rows * K * H][d] bf16: the dQ of each kept slot of a pass's rows, unscaled
  float *part;        // [max_parts][2][BS][d]: dV, dK (unscaled) of the items of shared buckets
  int64_t ntiles, nbk_g, nent_g, max_items, max_parts, tile;
  int32_t per_item;
  size_t total_bytes;
};

size_t ab_align(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of passes over at most `rows` query rows (the buckets, lists,
// slot dQ and item partials of one pass; D of every row).
AbWs ab_carve(const Dims &p, void *base, int64_t rows) {
  AbWs w;
  w.nent_g = rows * (int64_t)p.top_k;
  w.nbk_g = (int64_t)p.num_seqs * p.nb_max;
  w.tile = bucket_tile(w.nent_g, w.nbk_g);
  w.ntiles = (w.nent_g + w.tile - 1) / w.tile;
  w.per_item = kSteps * (kRows / (p.H / p.G));
  const int64_t nent = (int64_t)p.G * w.nent_g;
  // every bucket has one item more than its full items; a bucket with
  // partial slots has more than per_item entries
  w.max_items = nent / w.per_item + std::min<int64_t>((int64_t)p.G * w.nbk_g, nent) + 1;
  w.max_parts = 2 * (nent / w.per_item) + 1;
  size_t off = 0;
  char *c = static_cast<char *>(base);
  auto take = [&](size_t bytes) {
    char *r = c == nullptr ? nullptr : c + off;
    off += ab_align(bytes);
    return r;
  };
  w.cnt = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)p.G * w.ntiles * w.nbk_g));
  w.base = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  w.lists = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)nent));
  w.ibase = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  w.pbase = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  w.dsum = reinterpret_cast<float *>(take(sizeof(float) * (size_t)p.total_q * p.H));
  w.dq_part = reinterpret_cast<uint16_t *>(
      take(sizeof(uint16_t) * (size_t)nent / p.G * p.H * kD));
  w.part = reinterpret_cast<float *>(take(sizeof(float) * (size_t)w.max_parts * 2 * kBS * kD));
  w.total_bytes = off;
  return w;
}

__global__ __launch_bounds__(256) void ab_zero_kernel(float *__restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    x[i] = 0.f;
}

// One work-group per (group, sequence, block) bucket that no slot keeps:
// dk, dv <- 0 on its keys.  The keys of every other bucket are written by
// ab_item or ab_reduce.
__global__ __launch_bounds__(256) void ab_zero_unkept_kernel(const int32_t *__restrict__ base,
                                                             float *__restrict__ dk,
                                                             float *__restrict__ dv,
                                                             const int64_t *__restrict__ cu_kv,
                                                             int G, int nb_max, int64_t nbk_g) {
  const int64_t gb = blockIdx.x;
  if (base[gb + 1] != base[gb]) return;
  const int g = (int)(gb / nbk_g);
  const int64_t bkt = gb - (int64_t)g * nbk_g;
  const int b = (int)(bkt / nb_max), j = (int)(bkt - (int64_t)b * nb_max);
  const int64_t kv0 = cu_kv[b], lkv = cu_kv[b + 1] - kv0;
  const int64_t s0 = (int64_t)j * kBS;
  const int nkeys = (int)min<int64_t>(kBS, lkv - s0);  // <= 0 past the sequence's last block
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int x = threadIdx.x * 4; x < nkeys * kD; x += 256 * 4) {
    const int s = x / kD, c = x - s * kD;
    const int64_t o = ((kv0 + s0 + s) * G + g) * (int64_t)kD + c;
    *reinterpret_cast<f32x4 *>(dk + o) = z;
    *reinterpret_cast<f32x4 *>(dv + o) = z;
  }
}

// 16 lanes per (row, head), 8 channels each, then a 16-lane sum.
__global__ __launch_bounds__(256) void ab_dsum_kernel(const uint16_t *__restrict__ out,
                                                      const uint16_t *__restrict__ dout,
                                                      float *__restrict__ dsum, int64_t nrows) {
  const int64_t rh = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  float acc = 0.f;
  if (rh < nrows) {
    const u32x4 o = ld16(out + rh * kD + part * 8);
    const u32x4 g = ld16(dout + rh * kD + part * 8);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc = fmaf(bf16_lo(o[u]), bf16_lo(g[u]), acc);
      acc = fmaf(bf16_hi(o[u]), bf16_hi(g[u]), acc);
    }
  }
  acc += shfl_xor_f(acc, 8);
  acc += shfl_xor_f(acc, 4);
  acc += shfl_xor_f(acc, 2);
  acc += shfl_xor_f(acc, 1);
  if (part == 0 && rh < nrows) dsum[rh] = acc;
}


// LDS rows are padded so that every access pattern below is free of bank
// conflicts while each address is a per-lane base plus a compile-time
// offset (the loops' steps then cost no address arithmetic):
//  - rows of 128 bf16 (Q, dO, K, V) take 288 bytes, 8 banks apart: 8
//    consecutive rows reading 16 bytes of one column (MFMA operands, 8 lanes
//    per LDS cycle) cover 32 banks, and 4 consecutive rows reading 32 bytes
//    each (the transposing reads, 16 lanes per cycle) cover 32 banks;
//  - rows of 64 bf16 (P^T, dS^T) take 144 bytes, 36 banks apart: 16
//    consecutive rows writing 8 bytes, 8 rows reading 16 bytes and 4 rows
//    reading 32 bytes each fall on distinct banks.
constexpr int kRS = 144;  // elements per row of 128
constexpr int kPS = 72;   // elements per row of 64
__device__ __forceinline__ int off256(int r, int e) { return r * kRS + e; }
__device__ __forceinline__ int off128(int r, int e) { return r * kPS + e; }

// Transposing LDS read (ds_read_b64_tr_b16).  In each 16-lane group, lane i
// names a 4-element chunk; lane 4a + b receives element b of the chunks of
// lanes a, a + 4, a + 8 and a + 12.  So with lane i pointing at
// X[k0 + i / 4][n0 + 4 (i % 4)] of a row-major X, lane j receives
// X[k0 .. k0 + 3][n0 + j].
__device__ __forceinline__ u32x2 ld_tr(const uint16_t *p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)p);
  return __builtin_bit_cast(u32x2, r);
}
// MFMA 32x32x16 operand holding X[k0 + 8 hh .. k0 + 8 hh + 7][n0 + lane % 32]
// (hh = lane / 32) of a row-major X with padded rows (OFF = off256 or
// off128): two transposing reads of 4 rows each.
template <int (*OFF)(int, int)>
__device__ __forceinline__ u32x4 ld_op_tr(const uint16_t *x, int k0, int n0, int lane) {
  const int i = lane & 15, grp = lane >> 4;
  const int r = k0 + 8 * (grp >> 1) + (i >> 2), e = n0 + 16 * (grp & 1) + 4 * (i & 3);
  const u32x2 a = ld_tr(x + OFF(r, e)), b = ld_tr(x + OFF(r + 4, e));
  return u32x4{a[0], a[1], b[0], b[1]};
}

// One work-group per work item, 8 waves; wave wv has kg = wv % 4 and
// hf = wv / 4.  K and V of the block stay in LDS (row-major) for the whole
// item.  Per step (64 rows):
//   phase 1  S = Q K^T and dP = dO V^T for keys 32 kg .. and rows 32 hf ..,
//            then P and dS; P^T and dS^T go to LDS [key][row]
//   phase 2  dV^T += dO^T P and dK^T += Q^T dS for channels 64 hf .. 64 hf + 63
//            and keys 32 kg .. over all 64 rows (each (key, channel) has one
//            owner, so no cross-wave sum); dQ^T = K^T dS^T for channels
//            32 kg .. and rows 32 hf .. over all 128 keys -> the rows' slots
// The transposed operands (dO^T, Q^T, K^T, dS) come from the row-major LDS
// copies through transposing reads.  MFMA 32x32x16 layouts as in
// msa_common.hpp.  The next step's Q and dO rows load into registers during
// phase 2 and are staged after a third barrier (phase 2 still reads qs, os).
template <int HPG>
__global__ __launch_bounds__(kItemThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
ab_item_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
               const uint16_t *__restrict__ v, const uint16_t *__restrict__ dout,
               const float *__restrict__ lse, const float *__restrict__ dsum,
               const int32_t *__restrict__ base, const int32_t *__restrict__ ibase,
               const int32_t *__restrict__ pbase, const int32_t *__restrict__ lists,
               uint16_t *__restrict__ dq_part, float *__restrict__ dk, float *__restrict__ dv,
               float *__restrict__ part, const int64_t *__restrict__ cu_q,
               const int64_t *__restrict__ cu_kv, int G, int H, int K, int nb_max,
               int64_t nbuckets, int per_item, float scale, int64_t e_lo, int accumulate) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kBS * kRS];    // K [key][d]
  __shared__ __attribute__((aligned(16))) uint16_t vs[kBS * kRS];    // V [key][d]
  __shared__ __attribute__((aligned(16))) uint16_t qs[kRows * kRS];  // Q [row][d]
  __shared__ __attribute__((aligned(16))) uint16_t os[kRows * kRS];  // dO [row][d]
  __shared__ __attribute__((aligned(16))) uint16_t pt[kBS * kPS];    // P^T [key][row]
  __shared__ __attribute__((aligned(16))) uint16_t st_[kBS * kPS];   // dS^T [key][row]
  __shared__ __attribute__((aligned(16))) float m_lse[kRows];  // log2-domain LSE (+inf: no row)
  __shared__ __attribute__((aligned(16))) float m_d[kRows];    // D
  __shared__ __attribute__((aligned(16))) int32_t m_pos[kRows];  // position (-1: no row)
  __shared__ int32_t m_off[kRows];     // dQ slot row (-1: no row)
  __shared__ int32_t m_ent[2][kRows];  // list entries of the rows of steps st + 1, st + 2

  const int32_t w = (int32_t)blockIdx.x;
  if (w >= ibase[nbuckets]) return;  // past the last item
  int64_t lo = 0, hi = nbuckets - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (ibase[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int64_t gb = lo;  // g * nbk_g + b * nb_max + j
  const int32_t it = w - ibase[gb], nit = ibase[gb + 1] - ibase[gb];
  const int32_t n_b = base[gb + 1] - base[gb];
  const int32_t first = base[gb] + it * per_item, n = min(per_item, n_b - it * per_item);
  const int64_t nbk_g = nbuckets / G;
  const int g = (int)(gb / nbk_g);
  const int64_t bkt = gb - (int64_t)g * nbk_g;
  const int b = (int)(bkt / nb_max), j = (int)(bkt - (int64_t)b * nb_max);
  const int64_t kv0 = cu_kv[b], lkv = cu_kv[b + 1] - kv0;
  const int64_t q0 = cu_q[b], base_pos = lkv - (cu_q[b + 1] - q0);
  const int64_t s0 = (int64_t)j * kBS;
  const int nkeys = (int)min<int64_t>(kBS, lkv - s0);
  constexpr int hpg = HPG, E = kRows / HPG;
  const int nsteps = (n + E - 1) / E;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int kg = wv & 3, hf = wv >> 2;
  const int li = lane & 31, hh = lane >> 5;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // K and V of the block, zero past the sequence's keys
  {
    const int key = tid & 127;
    const int64_t roff = ((kv0 + s0 + min(key, nkeys - 1)) * G + g) * (int64_t)kD;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = (tid >> 7) + 4 * u;
      st16(&ks[off256(key, pc * 8)], key < nkeys ? ld16(k + roff + pc * 8) : zero4);
      st16(&vs[off256(key, pc * 8)], key < nkeys ? ld16(v + roff + pc * 8) : zero4);
    }
  }

  // Rows of a step: thread tid loads pieces tid % 8 and tid % 8 + 8 of row
  // tid / 8 of Q and dO, and the row's LSE and D.  The list entry
  // naming the row is read one step earlier still (by the first wave, into
  // the m_ent ring), so no load of a step waits for another; rows past the
  // item repeat its last entry (valid memory) and are switched off when
  // staged.
  const int r_me = tid & 63;            // row of the entry ring slot this thread fills
  const int r_ld = tid >> 3, pc0 = tid & 7;  // row and first piece this thread loads
  auto load_entry = [&](int st) { return lists[first + min(st * E + r_me / hpg, n - 1)]; };
  u32x4 fq[2], fo[2];
  float f_lse = 0.f, f_d = 0.f;
  int32_t f_e = 0;
  auto fetch = [&](int32_t e) {
    const int64_t t = e / K;
    // the entry's row is a query of this bucket's sequence for which block j is causal
    MSA_DCHECK(e >= 0 && t >= q0 && t < cu_q[b + 1] && base_pos + (t - q0) >= s0);
    const int h = g * hpg + r_ld % hpg;
    const int64_t roff = (t * H + h) * (int64_t)kD;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pc = pc0 + 8 * u;  // 8 lanes cover 128 contiguous bytes of the row
      fq[u] = ld16(q + roff + pc * 8);
      fo[u] = ld16(dout + roff + pc * 8);
    }
    f_lse = lse[t * H + h];
    f_d = dsum[t * H + h];
    f_e = e;
  };
  auto stage_rows = [&](int st) {  // Q, dO and the metadata
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pc = pc0 + 8 * u;
      st16(&qs[off256(r_ld, pc * 8)], fq[u]);
      st16(&os[off256(r_ld, pc * 8)], fo[u]);
    }
    if (pc0 == 0) {  // one of the row's 8 loading threads
      const bool ok = st * E + r_ld / hpg < n;
      const int64_t t = f_e / K;
      m_lse[r_ld] = ok ? f_lse * kLog2e : __builtin_inff();
      m_d[r_ld] = ok ? f_d : 0.f;
      m_pos[r_ld] = ok ? (int)(base_pos + (t - q0)) : -1;
      m_off[r_ld] = ok ? (f_e - (int32_t)e_lo) * H + g * hpg + r_ld % hpg : -1;
    }
  };

  // The wave's K operands of phase 1 stay in registers for the whole item
  // (one LDS read of them per item instead of one per step).
  __syncthreads();
  u32x4 kreg[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) kreg[x] = ld16(&ks[off256(32 * kg + li, 16 * x + 8 * hh)]);
  f32x16 acc_v[2], acc_k[2];  // dV^T, dK^T tiles [channel][key] of channels 64 hf ..
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_v[x][r] = acc_k[x][r] = 0.f;
  const float c2 = scale * kLog2e;
  const int64_t keypos = s0 + 32 * kg + li;

  int32_t f_e2 = 0;  // entry of row r_me in step st + 2 (first wave)
  if (nsteps > 0) {
    if (tid < 64) {
      m_ent[0][r_me] = load_entry(0);
      m_ent[1][r_me] = load_entry(1);
    }
    __syncthreads();
    fetch(m_ent[0][r_ld]);
    stage_rows(0);
  }
  for (int st = 0; st < nsteps; ++st) {
    __syncthreads();
    // phase 1: S and dP for rows 32 hf .., keys 32 kg ..
    f32x16 sacc, pacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const u32x4 aq = ld16(&qs[off256(32 * hf + li, 16 * x + 8 * hh)]);
      const u32x4 bk = kreg[x];
      const u32x4 ao = ld16(&os[off256(32 * hf + li, 16 * x + 8 * hh)]);
      const u32x4 bv = ld16(&vs[off256(32 * kg + li, 16 * x + 8 * hh)]);
      sacc = mfma32x32x16(as_bf16x8(aq), as_bf16x8(bk), sacc);
      pacc = mfma32x32x16(as_bf16x8(ao), as_bf16x8(bv), pacc);
    }
    // register 4 q4 + i holds row 32 hf + 8 q4 + 4 hh + i and key keypos
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int row = 32 * hf + 8 * q4 + 4 * hh;
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&m_lse[row]);
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&m_d[row]);
      const u32x4 p4 = ld16(&m_pos[row]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * q4 + i;
        // the hardware exp2 (weights below 2^-126 become 0, far below the
        // bf16 rounding P gets next; exp2(-inf) = 0 for rows past the item)
        const float pv = keypos > (int64_t)(int32_t)p4[i]
                             ? 0.f
                             : __builtin_amdgcn_exp2f(sacc[r] * c2 - l4[i]);
        sacc[r] = pv;
        pacc[r] = pv * (pacc[r] - d4[i]);
      }
    }
    const int my_off = m_off[32 * hf + li];  // dQ row of this lane, read before it is restaged
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int row = 32 * hf + 8 * q4 + 4 * hh;  // rows row .. row + 3
      const u32x2 pv = {pack_bf16x2(sacc[4 * q4], sacc[4 * q4 + 1]),
                        pack_bf16x2(sacc[4 * q4 + 2], sacc[4 * q4 + 3])};
      const u32x2 dsv = {pack_bf16x2(pacc[4 * q4], pacc[4 * q4 + 1]),
                         pack_bf16x2(pacc[4 * q4 + 2], pacc[4 * q4 + 3])};
      *reinterpret_cast<u32x2 *>(&pt[off128(32 * kg + li, row)]) = pv;
      *reinterpret_cast<u32x2 *>(&st_[off128(32 * kg + li, row)]) = dsv;
    }
    __syncthreads();
    if (st + 1 < nsteps) {
      fetch(m_ent[(st + 1) & 1][r_ld]);
      if (tid < 64) f_e2 = load_entry(st + 2);
    }
    // phase 2: dV^T += dO^T P, dK^T += Q^T dS (channels 64 hf .., keys 32 kg .., 64 rows)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const u32x4 bp = ld16(&pt[off128(32 * kg + li, 16 * x + 8 * hh)]);
      const u32x4 bs = ld16(&st_[off128(32 * kg + li, 16 * x + 8 * hh)]);
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const u32x4 ao = ld_op_tr<off256>(os, 16 * x, 64 * hf + 32 * y, lane);
        const u32x4 aq = ld_op_tr<off256>(qs, 16 * x, 64 * hf + 32 * y, lane);
        acc_v[y] = mfma32x32x16(as_bf16x8(ao), as_bf16x8(bp), acc_v[y]);
        acc_k[y] = mfma32x32x16(as_bf16x8(aq), as_bf16x8(bs), acc_k[y]);
      }
    }
    // dQ^T = K^T dS^T for channels 32 kg .., rows 32 hf .. (all 128 keys), two chains
    f32x16 qa0, qa1;
#pragma unroll
    for (int r = 0; r < 16; ++r) qa0[r] = qa1[r] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; x += 2) {
      const u32x4 a0 = ld_op_tr<off256>(ks, 16 * x, 32 * kg, lane);
      const u32x4 b0 = ld_op_tr<off128>(st_, 16 * x, 32 * hf, lane);
      const u32x4 a1 = ld_op_tr<off256>(ks, 16 * x + 16, 32 * kg, lane);
      const u32x4 b1 = ld_op_tr<off128>(st_, 16 * x + 16, 32 * hf, lane);
      qa0 = mfma32x32x16(as_bf16x8(a0), as_bf16x8(b0), qa0);
      qa1 = mfma32x32x16(as_bf16x8(a1), as_bf16x8(b1), qa1);
    }
    // lane holds row 32 hf + li, channels 32 kg + 8 (r / 4) + 4 hh + r % 4; the
    // slot buffer keeps them in that order (stored position 32 kg + 16 hh + r,
    // see dq_channel), so the lane's 16 values are 32 contiguous bytes
    if (my_off >= 0) {
      uint16_t *dst = dq_part + (int64_t)my_off * kD + 32 * kg + 16 * hh;
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        u32x4 val;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = 8 * hv + 2 * m;
          val[m] = pack_bf16x2(qa0[r] + qa1[r], qa0[r + 1] + qa1[r + 1]);
        }
        st16(dst + 8 * hv, val);
      }
    }
    if (st + 1 < nsteps) {
      __syncthreads();  // phase 2 reads qs / os (transposed): all waves are past it
      stage_rows(st + 1);
      if (tid < 64) m_ent[st & 1][r_me] = f_e2;  // the slot of step st + 2
    }
  }

  const int key = 32 * kg + li;
  if (key >= nkeys) return;
  float *dvp, *dkp;
  float kscale;
  if (nit == 1) {
    dvp = dv + ((kv0 + s0 + key) * G + g) * (int64_t)kD;
    dkp = dk + ((kv0 + s0 + key) * G + g) * (int64_t)kD;
    kscale = scale;
  } else {
    float *pp = part + (int64_t)(pbase[gb] + it) * 2 * kBS * kD;
    dvp = pp + key * kD;
    dkp = pp + (kBS + key) * kD;
    kscale = 1.f;
  }
  // lane holds key 32 kg + li, channels 64 hf + 32 y + 8 (r / 4) + 4 hh + r % 4
  // a pass after the first adds to the dk / dv of the earlier passes
  const bool add = accumulate != 0 && nit == 1;
#pragma unroll
  for (int y = 0; y < 2; ++y)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int dc = 64 * hf + 32 * y + 8 * q4 + 4 * hh;
      f32x4 vv = {acc_v[y][4 * q4], acc_v[y][4 * q4 + 1], acc_v[y][4 * q4 + 2],
                  acc_v[y][4 * q4 + 3]};
      f32x4 kk = {acc_k[y][4 * q4] * kscale, acc_k[y][4 * q4 + 1] * kscale,
                  acc_k[y][4 * q4 + 2] * kscale, acc_k[y][4 * q4 + 3] * kscale};
      if (add) {
        vv += *reinterpret_cast<const f32x4 *>(dvp + dc);
        kk += *reinterpret_cast<const f32x4 *>(dkp + dc);
      }
      *reinterpret_cast<f32x4 *>(dvp + dc) = vv;
      *reinterpret_cast<f32x4 *>(dkp + dc) = kk;
    }
}

// Per bucket of several items, kReduceSplit work-groups (each a share of
// the block's key rows): dv, dk = the items' partials added in item order
// (dk scaled).
constexpr int kReduceSplit = 8;
__global__ __launch_bounds__(256) void ab_reduce_kernel(const int32_t *__restrict__ ibase,
                                                        const int32_t *__restrict__ pbase,
                                                        const float *__restrict__ part,
                                                        float *__restrict__ dk,
                                                        float *__restrict__ dv,
                                                        const int64_t *__restrict__ cu_kv, int G,
                                                        int nb_max, int64_t nbk_g, float scale,
                                                        int accumulate) {
  const int64_t gb = blockIdx.x;
  const int32_t nit = ibase[gb + 1] - ibase[gb];
  if (nit <= 1) return;
  const int g = (int)(gb / nbk_g);
  const int64_t bkt = gb - (int64_t)g * nbk_g;
  const int b = (int)(bkt / nb_max), j = (int)(bkt - (int64_t)b * nb_max);
  const int64_t kv0 = cu_kv[b], lkv = cu_kv[b + 1] - kv0;
  const int64_t s0 = (int64_t)j * kBS;
  const int nkeys = (int)min<int64_t>(kBS, lkv - s0);
  const float *src = part + (int64_t)pbase[gb] * 2 * kBS * kD;
  constexpr int kShare = kBS * kD / kReduceSplit;  // floats of one work-group
  const int x0 = blockIdx.y * kShare;
  for (int x = x0 + threadIdx.x * 4; x < min(x0 + kShare, nkeys * kD); x += 256 * 4) {
    f32x4 av = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
    for (int32_t i = 0; i < nit; ++i) {
      av += *reinterpret_cast<const f32x4 *>(src + (int64_t)i * 2 * kBS * kD + x);
      ak += *reinterpret_cast<const f32x4 *>(src + (int64_t)i * 2 * kBS * kD + kBS * kD + x);
    }
    const int s = x / kD, c = x - s * kD;
    const int64_t o = ((kv0 + s0 + s) * G + g) * (int64_t)kD + c;
    ak *= scale;
    if (accumulate) {  // a pass after the first adds to the earlier passes' sums
      av += *reinterpret_cast<const f32x4 *>(dv + o);
      ak += *reinterpret_cast<const f32x4 *>(dk + o);
    }
    *reinterpret_cast<f32x4 *>(dv + o) = av;
    *reinterpret_cast<f32x4 *>(dk + o) = ak;
  }
}

// Channel of stored position pos of a dQ slot row: position 32 t + 16 h + 4 i
// + e holds channel 32 t + 8 i + 4 h + e (the MFMA result order of a lane).
__device__ __forceinline__ int dq_channel(int pos) {
  const int t = pos >> 5, h = (pos >> 4) & 1, i = (pos >> 2) & 3, e = pos & 3;
  return 32 * t + 8 * i + 4 * h + e;
}

// 16 lanes per (row, head), 8 channels each: dq = scale * sum over the row's
// kept slots (in slot order) of the slot's dQ.  Slots that are padding or
// whose block holds no causal key of the row add nothing.
__global__ __launch_bounds__(256) void ab_dq_kernel(const uint16_t *__restrict__ dq_part,
                                                    const int32_t *__restrict__ block_idx,
                                                    float *__restrict__ dq,
                                                    const int64_t *__restrict__ cu_q,
                                                    const int64_t *__restrict__ cu_kv,
                                                    int num_seqs, int H, int G, int K,
                                                    int64_t total_q, int nb_max, float scale,
                                                    int64_t row_lo, int64_t row_hi) {
  const int64_t rh = row_lo * H + (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (rh >= row_hi * H) return;
  const int part = threadIdx.x & 15;
  const int64_t row = rh / H;
  const int h = (int)(rh - row * H);
  const int g = h / (H / G);
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t pos = sq.base + (row - sq.q0);
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  const int32_t *bi = block_idx + ((int64_t)g * total_q + row) * K;
  for (int i = 0; i < K; ++i) {
    const int jb = bi[i];
    if (jb < 0 || jb >= nb_max || pos < 0 || (int64_t)jb * kBS > pos) continue;
    const u32x4 x = ld16(dq_part + ((((row - row_lo) * K + i) * H) + h) * (int64_t)kD + part * 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[2 * m] += bf16_lo(x[m]);
      acc[2 * m + 1] += bf16_hi(x[m]);
    }
  }
  // stored positions 8 part .. 8 part + 7 are two runs of 4 channels
  float *dst = dq + rh * kD;
  const f32x4 a = {acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale};
  const f32x4 c = {acc[4] * scale, acc[5] * scale, acc[6] * scale, acc[7] * scale};
  *reinterpret_cast<f32x4 *>(dst + dq_channel(8 * part)) = a;
  *reinterpret_cast<f32x4 *>(dst + dq_channel(8 * part + 4)) = c;
}

void zero_fill(float *x, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  const unsigned zg = (unsigned)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(ab_zero_kernel, dim3(zg), dim3(256), 0, s, x, n);
}

}  // namespace

MSA_DEBUG_COUNTER(attn_bwd)

bool attn_bwd_supported(const Dims &p) {
  const int hpg = p.G > 0 ? p.H / p.G : 0;
  return p.d == kD && p.B == kBS &&
         (hpg == 1 || hpg == 2 || hpg == 4 || hpg == 8 || hpg == 16);
}

// Fewest query rows per pass when the workspace is too small for one pass.
constexpr int64_t kMinPassRows = 256;

// With no query row the call only clears dk and dv, and needs no workspace.
size_t attn_bwd_workspace_bytes(const Dims &p, int64_t rows_per_pass) {
  return p.total_q > 0
             ? ab_carve(p, nullptr, std::max<int64_t>(1, std::min(rows_per_pass, p.total_q))).total_bytes
             : 0;
}

size_t attn_bwd_workspace_min_bytes(const Dims &p) { return attn_bwd_workspace_bytes(p, kMinPassRows); }

int64_t attn_bwd_rows_per_pass(const Dims &p, size_t workspace_bytes) {
  if (attn_bwd_workspace_bytes(p, p.total_q) <= workspace_bytes) return p.total_q;
  if (attn_bwd_workspace_bytes(p, kMinPassRows) > workspace_bytes) return 0;
  int64_t lo = std::min<int64_t>(kMinPassRows, p.total_q), hi = p.total_q;  // fits, does not
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (attn_bwd_workspace_bytes(p, mid) <= workspace_bytes) lo = mid; else hi = mid;
  }
  return lo;
}

// Rows [row_lo, row_hi) of the backward: bucket their kept slots, then the
// item, reduce and dQ kernels.  With `accumulate`, dk and dv (cleared before
// the first pass) get this pass's sums added; otherwise they are written.
namespace {
void bwd_pass(const Dims &p, const AbWs &w, int64_t row_lo, int64_t row_hi, bool accumulate,
              const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *block_idx,
              const float *lse, const uint16_t *dout, float *dq, float *dk, float *dv,
              hipStream_t s) {
  const int64_t e_lo = row_lo * p.top_k, e_hi = row_hi * p.top_k;
  const size_t hist_bytes = sizeof(int32_t) * (size_t)w.nbk_g;
  const int64_t ntiles = std::max<int64_t>(1, (e_hi - e_lo + w.tile - 1) / w.tile);
  hipLaunchKernelGGL(bk_count_kernel, dim3((unsigned)ntiles, p.G), dim3(256), hist_bytes, s,
                     block_idx, p.cu_q, p.cu_kv, w.cnt, nullptr, p.num_seqs, p.top_k, p.total_q,
                     e_lo, e_hi, p.nb_max, p.B, ntiles, w.nbk_g, w.tile);
  const int64_t ncol = (int64_t)p.G * w.nbk_g;
  hipLaunchKernelGGL(bk_colscan_kernel, dim3((unsigned)((ncol + 255) / 256)), dim3(256), 0, s,
                     w.cnt, w.base, w.ibase, w.pbase, p.G, ntiles, w.nbk_g, w.per_item);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.base, ncol);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.ibase, ncol);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.pbase, ncol);
  hipLaunchKernelGGL(bk_scatter_kernel, dim3((unsigned)ntiles, p.G), dim3(64), hist_bytes, s,
                     block_idx, p.cu_q, p.cu_kv, w.cnt, w.base, w.lists, p.num_seqs, p.top_k,
                     p.total_q, e_lo, e_hi, p.nb_max, p.B, ntiles, w.nbk_g, w.tile);
  profile_mark(s);
  if (!accumulate)
    hipLaunchKernelGGL(ab_zero_unkept_kernel, dim3((unsigned)ncol), dim3(256), 0, s, w.base, dk,
                       dv, p.cu_kv, p.G, p.nb_max, w.nbk_g);
  profile_mark(s);
  const int acc = accumulate ? 1 : 0;
  auto item = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)w.max_items), dim3(kItemThreads), 0, s, q, k, v, dout,
                       lse, w.dsum, w.base, w.ibase, w.pbase, w.lists, w.dq_part, dk, dv, w.part,
                       p.cu_q, p.cu_kv, p.G, p.H, p.top_k, p.nb_max, ncol, w.per_item, p.scale,
                       e_lo, acc);
  };
  switch (p.H / p.G) {
    case 1: item(ab_item_kernel<1>); break;
    case 2: item(ab_item_kernel<2>); break;
    case 4: item(ab_item_kernel<4>); break;
    case 8: item(ab_item_kernel<8>); break;
    default: item(ab_item_kernel<16>); break;
  }
  profile_mark(s);
  hipLaunchKernelGGL(ab_reduce_kernel, dim3((unsigned)ncol, kReduceSplit), dim3(256), 0, s,
                     w.ibase, w.pbase, w.part, dk, dv, p.cu_kv, p.G, p.nb_max, w.nbk_g, p.scale,
                     acc);
  profile_mark(s);
  const int64_t nrh = (row_hi - row_lo) * p.H;
  hipLaunchKernelGGL(ab_dq_kernel, dim3((unsigned)((nrh + 15) / 16)), dim3(256), 0, s,
                     w.dq_part, block_idx, dq, p.cu_q, p.cu_kv, p.num_seqs, p.H, p.G, p.top_k,
                     p.total_q, p.nb_max, p.scale, row_lo, row_hi);
  profile_mark(s);
}
}  // namespace

hipError_t launch_attn_bwd_bf16(const Dims &p, const uint16_t *q, const uint16_t *k,
                                const uint16_t *v, const int32_t *block_idx, const uint16_t *out,
                                const float *lse, const uint16_t *dout, float *dq, float *dk,
                                float *dv, void *workspace, int64_t rows_per_pass, hipStream_t s) {
  if (p.total_q == 0 || p.total_kv == 0) {  // nothing kept: all gradients are 0
    zero_fill(dk, p.total_kv * p.G * (int64_t)kD, s);
    zero_fill(dv, p.total_kv * p.G * (int64_t)kD, s);
    zero_fill(dq, p.total_q * p.H * (int64_t)kD, s);
    profile_mark(s);
    return hipGetLastError();
  }
  if (rows_per_pass <= 0) return hipErrorInvalidValue;
  const AbWs w = ab_carve(p, workspace, rows_per_pass);
  const int64_t nrows = p.total_q * p.H;
  hipLaunchKernelGGL(ab_dsum_kernel, dim3((unsigned)((nrows + 15) / 16)), dim3(256), 0, s, out,
                     dout, w.dsum, nrows);
  profile_mark(s);
  const bool passes = rows_per_pass < p.total_q;
  if (passes) {  // every pass adds its sums
    zero_fill(dk, p.total_kv * p.G * (int64_t)kD, s);
    zero_fill(dv, p.total_kv * p.G * (int64_t)kD, s);
  }
  for (int64_t r0 = 0; r0 < p.total_q; r0 += rows_per_pass) {
    bwd_pass(p, w, r0, std::min(p.total_q, r0 + rows_per_pass), passes, q, k, v, block_idx, lse,
             dout, dq, dk, dv, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace msa
