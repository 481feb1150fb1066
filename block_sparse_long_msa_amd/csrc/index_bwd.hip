// Backward of the Index Branch max-pooling ("MiniMax Sparse Attention" page,
// Summary, paragraph 2: a block's score is the maximum of token-level
// index-query / index-key dot products, so the gradient of a kept block's
// score reaches only the causal key that attains that maximum).  Given the
// gradient c[g, r, i] of every kept slot's score (for instance the indexer KL
// gradient), with a = the arg-max key of block block_idx[g, r, i] for row r:
//   dq_idx[r, g] = sum over slots i (in slot order) of c[g,r,i] * k_idx[a, g]
//   dk_idx[s, g] = sum over (r, i) with a = s (in (r, i) order) of c[g,r,i] * q_idx[r, g]
// The arg-max is an integer decided by floating point: each key's dot
// product is summed in fp32 (bf16 inputs on the matrix cores, whose bf16
// products are exact in fp32; fp32 inputs in channel order, every product
// rounded to fp32 before it is added), and ties go to the lower key.  Any
// fp32 summation order is within the same rounding bound of the exact dot
// product, so keys whose products differ by less than that bound may swap.
//
// Deterministic, without floating-point atomics:
//   ib_zero      dk_idx <- 0 (keys no slot takes keep 0)
//   bk_count, bk_colscan, bk_basescan, bk_scatter (buckets.hpp): the list of
//                every bucket (sequence, block) in (row, slot) order, split
//                into items of kIE entries; invalid slots get arg-max -1
//   ib_item      per work item (at most kIE consecutive entries of one
//                bucket's list, so popular blocks are shared out): for each
//                entry in list order the arg-max over the causal keys (bf16:
//                S^T = K Q^T tiles on the matrix cores from the block's keys
//                staged once in LDS; fp32: key operands in scalar
//                registers), then each key row sums
//                c * q_idx over the entries that chose it, in list order.  A
//                bucket of one item writes dk_idx; the items of a larger
//                bucket write partial sums.  The arg-max is stored for ib_dq.
//   ib_reduce    per bucket of several items: dk_idx = the items' partial
//                sums added in item order
//   ib_dq        per (group, row): dq_idx from the stored arg-max keys
#include <algorithm>
#include <type_traits>

#include "launch.hpp"
#include "buckets.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kIE = 1024;  // entries per work item of the arg-max pass

struct IbWs {
  int32_t *cnt;    // [G][ntiles][nbk_g]: tile counts, then exclusive tile offsets
  int32_t *base;   // [G * nbk_g + 1]: bucket totals, then exclusive starts
  int32_t *lists;  // [G * total_q * K] entries e = row * K + slot, grouped by bucket
  int32_t *amax;   // [G][total_q][K] arg-max key (packed key row) or -1
  int32_t *ibase;  // [G * nbk_g + 1]: items per bucket, then exclusive item starts
  int32_t *pbase;  // [G * nbk_g + 1]: partial slots per bucket (its items if > 1)
  float *part;     // [max_parts][BS][d_idx] key-side partial sums of shared buckets
  int64_t ntiles, nbk_g, nent_g, max_items, max_parts, tile;
  size_t total_bytes;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

IbWs ib_carve(const Dims &p, void *base) {
  IbWs w;
  w.nent_g = p.total_q * (int64_t)p.top_k;
  w.nbk_g = (int64_t)p.num_seqs * p.nb_max;
  w.tile = bucket_tile(w.nent_g, w.nbk_g);
  w.ntiles = (w.nent_g + w.tile - 1) / w.tile;
  size_t off = 0;
  char *c = static_cast<char *>(base);
  auto take = [&](size_t bytes) {
    char *r = c == nullptr ? nullptr : c + off;
    off += al256(bytes);
    return reinterpret_cast<int32_t *>(r);
  };
  w.cnt = take(sizeof(int32_t) * (size_t)p.G * w.ntiles * w.nbk_g);
  w.base = take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1));
  w.lists = take(sizeof(int32_t) * (size_t)p.G * w.nent_g);
  w.amax = take(sizeof(int32_t) * (size_t)p.G * w.nent_g);
  w.ibase = take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1));
  w.pbase = take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1));
  // every bucket has one item more than its full kIE-entry items; a bucket
  // with partial slots has more than kIE entries
  const int64_t nent = (int64_t)p.G * w.nent_g;
  w.max_items = nent / kIE + std::min<int64_t>((int64_t)p.G * w.nbk_g, nent) + 1;
  w.max_parts = 2 * (nent / kIE) + 1;
  w.part = reinterpret_cast<float *>(take(sizeof(float) * (size_t)w.max_parts * p.B * p.d_idx));
  w.total_bytes = off;
  return w;
}

__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// One step of the fp32 arg-max dot product: acc + q * k with the product
// rounded to fp32 before the add (contraction switched off).
__device__ __forceinline__ float dot_step(float acc, float q, float k) {
#pragma clang fp contract(off)
  return acc + q * k;
}

__global__ __launch_bounds__(256) void ib_zero_kernel(float *__restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    x[i] = 0.f;
}

// One work-group per work item: entries [it * kIE, min(n, (it + 1) * kIE))
// of one bucket's list.  The item's rows and score gradients are staged in
// LDS first; the index queries of each 64-entry chunk are loaded into
// registers while the chunk before it is processed (two LDS buffers, bf16
// kept as bf16).  For bf16 the block's index keys are staged in LDS once and
// the arg-max runs on the matrix cores; for fp32 the keys are read with
// scalar loads, lane x handling entry x of a chunk in every wave and the
// waves splitting the keys.  For the key-side sum, the TPR threads of key row
// s each own DI / TPR of its channels.
template <typename T, int DI, int BS>
__global__ __launch_bounds__(256) void ib_item_kernel(
    const T *__restrict__ q_idx, const T *__restrict__ k_idx, const float *__restrict__ grad,
    const int32_t *__restrict__ base, const int32_t *__restrict__ ibase,
    const int32_t *__restrict__ pbase, const int32_t *__restrict__ lists,
    int32_t *__restrict__ amax, float *__restrict__ dk_idx, float *__restrict__ part,
    const int64_t *__restrict__ cu_q, const int64_t *__restrict__ cu_kv, int G, int K,
    int64_t total_q, int nb_max, int64_t nbuckets) {
  constexpr bool BF = sizeof(T) == 2;    // bf16: arg-max on the matrix cores
  using QE = std::conditional_t<BF, uint16_t, float>;  // element of the staged queries
  constexpr int TPR = 256 / BS;          // threads per key row (2 or 4)
  constexpr int CPT = DI / TPR;          // channels per thread in the key-side sum
  constexpr int KS = BF ? DI + 8 : DI + 4;  // padded LDS row of the chunk's queries (16-byte rows)
  constexpr int EPP = 16 / (int)sizeof(T);         // elements per 16-byte piece
  constexpr int PPR = DI / EPP;                    // pieces per query row
  constexpr int PPT = (64 * PPR + 255) / 256;      // pieces per thread and chunk
  constexpr int KR = DI + 8;             // padded LDS row of the block's index keys (bf16)
  typedef uint32_t piece_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) QE qs[2][64 * KS];  // index queries of a chunk's entries
  __shared__ __attribute__((aligned(16))) uint16_t kst[BF ? BS * KR : 8];  // the block's index keys
  __shared__ int32_t ent_row[kIE];       // the item's rows
  __shared__ float ent_c[kIE];           // and score gradients
  __shared__ int32_t as_[64];            // arg-max of the chunk's entries (-1 none)
  __shared__ float bv[256];              // arg-max candidates of the 4 waves
  __shared__ int32_t bs[256];
  const int32_t w = (int32_t)blockIdx.x;
  if (w >= ibase[nbuckets]) return;      // past the last item
  // the bucket holding item w: the last one whose first item is <= w
  int64_t lo = 0, hi = nbuckets - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (ibase[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int64_t gb = lo;                 // g * nbk_g + b * nb_max + j
  const int32_t it = w - ibase[gb], nit = ibase[gb + 1] - ibase[gb];
  const int32_t n_b = base[gb + 1] - base[gb];
  const int32_t first = base[gb] + it * kIE, n = min(kIE, n_b - it * kIE);
  const int64_t nbk_g = nbuckets / G;
  const int g = (int)(gb / nbk_g);
  const int64_t bkt = gb - (int64_t)g * nbk_g;
  const int b = (int)(bkt / nb_max), j = (int)(bkt - (int64_t)b * nb_max);
  const int64_t kv0 = cu_kv[b], lkv = cu_kv[b + 1] - kv0;
  const int64_t q0 = cu_q[b], base_pos = lkv - (cu_q[b + 1] - q0);
  const int64_t s0 = (int64_t)j * BS;
  const int nkeys = (int)min<int64_t>(BS, lkv - s0);
  const int tid = threadIdx.x;
  const int64_t nent = total_q * K;
  for (int x = tid; x < n; x += 256) {
    const int32_t e = lists[first + x];
    const int64_t row = e / K;
    // the entry's row is a query of this bucket's sequence for which block j is causal
    MSA_DCHECK(e >= 0 && row >= q0 && row < cu_q[b + 1] && base_pos + (row - q0) >= s0);
    ent_row[x] = (int32_t)row;
    ent_c[x] = grad[(int64_t)g * nent + e];
  }
  __syncthreads();
  // index-query pieces of chunk c0: piece pc = tid + 256 u is entry pc / PPR,
  // elements EPP * (pc % PPR) ..; entries past the item read its last entry
  piece_t pf[PPT];
  auto prefetch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int pc = min(tid + 256 * u, 64 * PPR - 1);
      const int xe = min(c0 + pc / PPR, n - 1);
      pf[u] = *reinterpret_cast<const piece_t *>(
          q_idx + ((int64_t)ent_row[xe] * G + g) * DI + EPP * (pc % PPR));
    }
  };
  auto stash = [&](QE *dst) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int pc = tid + 256 * u;
      if (PPT * 256 != 64 * PPR && pc >= 64 * PPR) break;
      const int xe = pc / PPR, c = EPP * (pc % PPR);
      if constexpr (BF) {
        *reinterpret_cast<piece_t *>(&dst[xe * KS + c]) = pf[u];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[xe * KS + c + i] = __uint_as_float(pf[u][i]);
      }
    }
  };
  const int srow = tid / TPR, c_lo = (tid % TPR) * CPT;
  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
  if constexpr (BF) {
    // the block's index keys, rows past the sequence's keys read its last key
    // (an entry's causal limit never reaches them)
    constexpr int KP = BS * DI / 8;  // 16-byte pieces of the block
    for (int pc = tid; pc < KP; pc += 256) {
      const int r = pc / (DI / 8), c = 8 * (pc % (DI / 8));
      const T *src = k_idx + ((kv0 + s0 + min(r, nkeys - 1)) * G + g) * (int64_t)DI + c;
      *reinterpret_cast<piece_t *>(&kst[r * KR + c]) = *reinterpret_cast<const piece_t *>(src);
    }
  }
  prefetch(0);
  stash(qs[0]);
  for (int32_t c0 = 0, buf = 0; c0 < n; c0 += 64, buf ^= 1) {
    const int cn = min(64, n - c0);
    __syncthreads();  // qs[buf] is filled; the previous chunk's as_ / bv are consumed
    if (c0 + 64 < n) prefetch(c0 + 64);
    if constexpr (BF) {
      // arg-max on the matrix cores: S^T = K Q^T tiles of 32 keys x 32
      // entries (bf16 products are exact in fp32, sums in fp32).  The
      // (key tile, entry tile) pairs are dealt to the waves; a lane ends with
      // the best of its 16 keys for entry 32 et + lane % 32 (keys in
      // increasing order, the lower key on a tie), then the two halves of the
      // wave combine.  Keys past an entry's causal limit are ignored.
      constexpr int NKT = BS / 32, NU = NKT * 2, UPW = NU / 4;  // units per wave
      const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
      const int li = lane & 31, hh = lane >> 5;
#pragma unroll
      for (int uu = 0; uu < UPW; ++uu) {
        const int unit = wv * UPW + uu, kt = unit % NKT, et = unit / NKT;
        f32x16 sc = f32x16{};
#pragma unroll
        for (int x = 0; x < DI / 16; ++x) {
          const u32x4 ak = *reinterpret_cast<const u32x4 *>(&kst[(32 * kt + li) * KR + 16 * x + 8 * hh]);
          const u32x4 bq = *reinterpret_cast<const u32x4 *>(&qs[buf][(32 * et + li) * KS + 16 * x + 8 * hh]);
          sc = mfma32x32x16(as_bf16x8(ak), as_bf16x8(bq), sc);
        }
        const int xe = 32 * et + li;  // the lane's entry
        const int lim = xe < cn ? (int)min<int64_t>(nkeys, base_pos + (ent_row[c0 + xe] - q0) - s0 + 1) : 0;
        float best = neg_inf();
        int bsel = -1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {  // key 32 kt + 8 (r / 4) + 4 hh + r % 4, increasing in r
          const int key = 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key < lim && (bsel < 0 || sc[r] > best)) {
            best = sc[r];
            bsel = key;
          }
        }
        const float ob = shfl_xor_f(best, 32);
        const int os = __shfl_xor(bsel, 32, 64);
        if (os >= 0 && (bsel < 0 || ob > best || (ob == best && os < bsel))) {
          best = ob;
          bsel = os;
        }
        if (hh == 0) {
          bv[64 * kt + xe] = best;
          bs[64 * kt + xe] = bsel;
        }
      }
    } else {
      // fp32 inputs: lane x of every wave holds entry x's index query in registers;
      // wave wv takes keys wv, wv + 4, ..., so all lanes of a wave need the same
      // key element, which comes from global memory at a wave-uniform address
      // into scalar registers.  Four keys' sums run at a time as independent
      // chains; each sum still runs in channel order.  Keys past an entry's
      // causal limit are computed and ignored.
      {
        const int x = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        // causal keys of the block for entry x's row
        const int lim = x < cn ? (int)min<int64_t>(nkeys, base_pos + (ent_row[c0 + x] - q0) - s0 + 1) : 0;
        float best = neg_inf();
        int bsel = -1;
        float qr[DI];
#pragma unroll
        for (int c = 0; c < DI; c += 4) {
          const float4 v = *reinterpret_cast<const float4 *>(&qs[buf][x * KS + c]);
          qr[c] = v.x;
          qr[c + 1] = v.y;
          qr[c + 2] = v.z;
          qr[c + 3] = v.w;
        }
        for (int s = wv; s < nkeys; s += 16) {
          float d[4] = {0.f, 0.f, 0.f, 0.f};
          // the four key rows, read from global memory at wave-uniform
          // addresses (scalar loads; rows past the block's end read its last row)
          const T *kr[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            kr[u] = k_idx + ((kv0 + s0 + min(s + 4 * u, nkeys - 1)) * G + g) * (int64_t)DI;
          // 16 channels of the four rows at a time (a scheduling barrier keeps
          // the compiler from hoisting further scalar loads): a modest number
          // of scalar registers in flight
#pragma unroll
          for (int c = 0; c < DI; c += 4) {
            if (c % 16 == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float4 kv = *reinterpret_cast<const float4 *>(kr[u] + c);
              d[u] = dot_step(d[u], qr[c], kv.x);
              d[u] = dot_step(d[u], qr[c + 1], kv.y);
              d[u] = dot_step(d[u], qr[c + 2], kv.z);
              d[u] = dot_step(d[u], qr[c + 3], kv.w);
            }
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {  // keys in increasing order; past the limit ignored
            if (s + 4 * u < lim && (d[u] > best || bsel < 0)) {
              best = d[u];
              bsel = s + 4 * u;
            }
          }
        }
        bv[tid] = best;
        bs[tid] = bsel;
      }
    }
    __syncthreads();
    if (tid < cn) {
      float best = bv[tid];
      int bsel = bs[tid];
      constexpr int NCAND = BF ? BS / 32 : 4;  // candidates per entry: key tiles, or waves
      for (int u = 1; u < NCAND; ++u) {  // the larger value; the lower key on a tie
        const float v = bv[64 * u + tid];
        const int s = bs[64 * u + tid];
        if (s >= 0 && (bsel < 0 || v > best || (v == best && s < bsel))) {
          best = v;
          bsel = s;
        }
      }
      as_[tid] = bsel;
      amax[(int64_t)g * nent + lists[first + c0 + tid]] = bsel < 0 ? -1 : (int32_t)(kv0 + s0 + bsel);
    }
    __syncthreads();
    // key side: row srow adds c * q over the chunk's entries that chose it,
    // in entry order.  A wave owns rows [wv * 64 / TPR, (wv + 1) * 64 / TPR):
    // lane x reads entry x's arg-max, and the wave visits only the entries
    // whose arg-max it owns, lowest first.
    {
      const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
      const int my_a = lane < cn ? as_[lane] : -1;
      const int r_lo = wv * (64 / TPR);
      uint64_t m = ballot64(my_a >= r_lo && my_a < r_lo + 64 / TPR);
      while (m != 0) {
        const int x = (int)__builtin_ctzll(m);
        m &= m - 1;
        const int r = __builtin_amdgcn_readlane(my_a, x);
        if (srow == r) {
          const float cx = ent_c[c0 + x];
#pragma unroll
          for (int c = 0; c < CPT; c += 4) {
            float4 v;
            if constexpr (BF) {
              const u32x2 w2 = *reinterpret_cast<const u32x2 *>(&qs[buf][x * KS + c_lo + c]);
              v = float4{bf16_lo(w2.x), bf16_hi(w2.x), bf16_lo(w2.y), bf16_hi(w2.y)};
            } else {
              v = *reinterpret_cast<const float4 *>(&qs[buf][x * KS + c_lo + c]);
            }
            acc[c] = fmaf(cx, v.x, acc[c]);
            acc[c + 1] = fmaf(cx, v.y, acc[c + 1]);
            acc[c + 2] = fmaf(cx, v.z, acc[c + 2]);
            acc[c + 3] = fmaf(cx, v.w, acc[c + 3]);
          }
        }
      }
    }
    if (c0 + 64 < n) stash(qs[buf ^ 1]);
  }
  if (nit == 1) {
    if (srow < nkeys) {
      float *dst = dk_idx + ((kv0 + s0 + srow) * G + g) * (int64_t)DI + c_lo;
#pragma unroll
      for (int c = 0; c < CPT; ++c) dst[c] = acc[c];
    }
  } else {
    float *dst = part + ((int64_t)(pbase[gb] + it) * BS + srow) * DI + c_lo;
#pragma unroll
    for (int c = 0; c < CPT; ++c) dst[c] = acc[c];
  }
}

// One work-group per bucket; only buckets of several items do work: each
// key-row channel adds the items' partial sums in item order.
template <int DI, int BS>
__global__ __launch_bounds__(256) void ib_reduce_kernel(const int32_t *__restrict__ ibase,
                                                        const int32_t *__restrict__ pbase,
                                                        const float *__restrict__ part,
                                                        float *__restrict__ dk_idx,
                                                        const int64_t *__restrict__ cu_kv, int G,
                                                        int nb_max, int64_t nbk_g) {
  const int64_t gb = blockIdx.x;
  const int32_t nit = ibase[gb + 1] - ibase[gb];
  if (nit <= 1) return;
  const int g = (int)(gb / nbk_g);
  const int64_t bkt = gb - (int64_t)g * nbk_g;
  const int b = (int)(bkt / nb_max), j = (int)(bkt - (int64_t)b * nb_max);
  const int64_t kv0 = cu_kv[b], lkv = cu_kv[b + 1] - kv0;
  const int64_t s0 = (int64_t)j * BS;
  const int nkeys = (int)min<int64_t>(BS, lkv - s0);
  const float *src = part + (int64_t)pbase[gb] * BS * DI;
  for (int x = threadIdx.x; x < nkeys * DI; x += 256) {
    float acc = 0.f;
    for (int32_t i = 0; i < nit; ++i) acc += src[(int64_t)i * BS * DI + x];
    const int s = x / DI, c = x - s * DI;
    dk_idx[((kv0 + s0 + s) * G + g) * (int64_t)DI + c] = acc;
  }
}

// One wave per (group, row): dq_idx[row, g] = sum over slots (in order) of
// c * k_idx[arg-max key]; lanes hold channels.
template <typename T, int DI>
__global__ __launch_bounds__(256) void ib_dq_kernel(const T *__restrict__ k_idx,
                                                    const float *__restrict__ grad,
                                                    const int32_t *__restrict__ amax,
                                                    float *__restrict__ dq_idx, int G, int K,
                                                    int64_t total_q,
                                                    [[maybe_unused]] int64_t total_kv) {
  constexpr int CPL = (DI + 63) / 64;  // channels per lane
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= total_q) return;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t rk = ((int64_t)g * total_q + row) * K;
  // lane i holds slot i's arg-max and gradient; the slots are then taken in
  // order, four key rows requested before any is used (a slot without an
  // arg-max reads key row 0 with weight 0)
  const int32_t am = lane < K ? amax[rk + lane] : -1;
  MSA_DCHECK(am < total_kv);
  const float gc = lane < K ? grad[rk + lane] : 0.f;
  float acc[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) acc[u] = 0.f;
  for (int i0 = 0; i0 < K; i0 += 4) {
    float kv[4][CPL], c[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = min(i0 + v, K - 1);
      const int32_t a = __builtin_amdgcn_readlane(am, i);
      c[v] = (i0 + v < K && a >= 0) ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gc), i)) : 0.f;
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int ch = min(lane + 64 * u, DI - 1);
        kv[v][u] = to_f32(k_idx[((int64_t)max(a, 0) * G + g) * DI + ch]);
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int u = 0; u < CPL; ++u) acc[u] = fmaf(c[v], kv[v][u], acc[u]);
  }
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int ch = lane + 64 * u;
    if (ch < DI) dq_idx[(row * G + g) * (int64_t)DI + ch] = acc[u];
  }
}

template <typename T, int DI, int BS>
hipError_t launch_ib(const Dims &p, const T *q_idx, const T *k_idx, const int32_t *block_idx,
                     const float *grad, float *dq_idx, float *dk_idx, void *workspace,
                     hipStream_t s) {
  IbWs w = ib_carve(p, workspace);
  const int64_t nk = p.total_kv * p.G * (int64_t)DI;
  if (nk > 0) {
    const unsigned zg = (unsigned)std::min<int64_t>((nk + 255) / 256, 65536);
    hipLaunchKernelGGL(ib_zero_kernel, dim3(zg), dim3(256), 0, s, dk_idx, nk);
  }
  profile_mark(s);
  const size_t hist_bytes = sizeof(int32_t) * (size_t)w.nbk_g;
  hipLaunchKernelGGL(bk_count_kernel, dim3((unsigned)w.ntiles, p.G), dim3(256), hist_bytes, s,
                     block_idx, p.cu_q, p.cu_kv, w.cnt, w.amax, p.num_seqs, p.top_k, p.total_q,
                     (int64_t)0, w.nent_g, p.nb_max, p.B, w.ntiles, w.nbk_g, w.tile);
  profile_mark(s);
  const int64_t ncol = (int64_t)p.G * w.nbk_g;
  hipLaunchKernelGGL(bk_colscan_kernel, dim3((unsigned)((ncol + 255) / 256)), dim3(256), 0, s,
                     w.cnt, w.base, w.ibase, w.pbase, p.G, w.ntiles, w.nbk_g, kIE);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.base, ncol);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.ibase, ncol);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.pbase, ncol);
  profile_mark(s);
  hipLaunchKernelGGL(bk_scatter_kernel, dim3((unsigned)w.ntiles, p.G), dim3(64), hist_bytes, s,
                     block_idx, p.cu_q, p.cu_kv, w.cnt, w.base, w.lists, p.num_seqs, p.top_k,
                     p.total_q, (int64_t)0, w.nent_g, p.nb_max, p.B, w.ntiles, w.nbk_g, w.tile);
  profile_mark(s);
  hipLaunchKernelGGL((ib_item_kernel<T, DI, BS>), dim3((unsigned)w.max_items), dim3(256), 0, s,
                     q_idx, k_idx, grad, w.base, w.ibase, w.pbase, w.lists, w.amax, dk_idx, w.part,
                     p.cu_q, p.cu_kv, p.G, p.top_k, p.total_q, p.nb_max, ncol);
  profile_mark(s);
  hipLaunchKernelGGL((ib_reduce_kernel<DI, BS>), dim3((unsigned)ncol), dim3(256), 0, s, w.ibase,
                     w.pbase, w.part, dk_idx, p.cu_kv, p.G, p.nb_max, w.nbk_g);
  profile_mark(s);
  hipLaunchKernelGGL((ib_dq_kernel<T, DI>), dim3((unsigned)((p.total_q + 3) / 4), p.G), dim3(256),
                     0, s, k_idx, grad, w.amax, dq_idx, p.G, p.top_k, p.total_q, p.total_kv);
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace

MSA_DEBUG_COUNTER(index_bwd)

size_t index_bwd_workspace_bytes(const Dims &p) {
  return p.total_q > 0 ? ib_carve(p, nullptr).total_bytes : 0;
}

int64_t index_bwd_hist_bytes(const Dims &p) {
  return (int64_t)sizeof(int32_t) * p.num_seqs * (int64_t)p.nb_max;
}

hipError_t launch_index_bwd(const Dims &p, bool bf16, const void *q_idx, const void *k_idx,
                            const int32_t *block_idx, const float *grad, float *dq_idx,
                            float *dk_idx, void *workspace, hipStream_t s) {
  if (p.total_q <= 0 || p.total_kv <= 0) {  // no slot takes a key: zero gradients
    const int64_t nk = p.total_kv * p.G * (int64_t)p.d_idx;
    const int64_t nq = p.total_q * p.G * (int64_t)p.d_idx;
    if (nk > 0)
      hipLaunchKernelGGL(ib_zero_kernel, dim3((unsigned)std::min<int64_t>((nk + 255) / 256, 65536)),
                         dim3(256), 0, s, dk_idx, nk);
    if (nq > 0)
      hipLaunchKernelGGL(ib_zero_kernel, dim3((unsigned)std::min<int64_t>((nq + 255) / 256, 65536)),
                         dim3(256), 0, s, dq_idx, nq);
    profile_mark(s);
    return hipGetLastError();
  }
#define MSA_IB_CASE(DI_, BS_)                                                                    \
  if (p.d_idx == DI_ && p.B == BS_) {                                                            \
    if (bf16)                                                                                    \
      return launch_ib<uint16_t, DI_, BS_>(p, static_cast<const uint16_t *>(q_idx),              \
                                           static_cast<const uint16_t *>(k_idx), block_idx,      \
                                           grad, dq_idx, dk_idx, workspace, s);                  \
    return launch_ib<float, DI_, BS_>(p, static_cast<const float *>(q_idx),                      \
                                      static_cast<const float *>(k_idx), block_idx, grad,        \
                                      dq_idx, dk_idx, workspace, s);                             \
  }
  MSA_IB_CASE(32, 64) MSA_IB_CASE(32, 128) MSA_IB_CASE(64, 64) MSA_IB_CASE(64, 128)
  MSA_IB_CASE(128, 64) MSA_IB_CASE(128, 128)
#undef MSA_IB_CASE
  return hipErrorInvalidValue;
}

}  // namespace msa
