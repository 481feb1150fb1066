// Index Branch block scoring ("MiniMax Sparse Attention" page, Summary,
// paragraph 2): every key/value block is scored by max-pooling the
// token-level dot products of a query's index vector with the block's index
// keys.  scores[g, row, j] = max over causal keys s of block j of
// <q_idx[row, g], k_idx[s, g]>, and -inf where block j holds no causal key.
//
// Three kernels:
//  * index_score_mfma_kernel  - bf16 prefill.  A work-group (8 waves) owns 512
//    queries x 16 key blocks of one (sequence, group).  The index queries stay in
//    registers as MFMA B operands for the whole work-group; key blocks stream
//    through a two-stage LDS ring, filled by direct global-to-LDS loads one
//    block ahead (XOR-swizzled 16-byte chunks keep the operand reads free of
//    bank conflicts); each wave computes S^T = K * Q^T tiles (keys x queries)
//    with 32x32x16 bf16 MFMA so a lane holds 16 keys of ONE query column and
//    the block max is an in-lane max chain plus one cross-half lane swap.  Causal
//    masking is applied only to blocks that can hold keys past a query's
//    position, in a separate loop.
//  * index_score_decode_kernel - bf16, one query per sequence: a streaming
//    scan of the index-key cache (HBM-bound).  Lanes read consecutive 16-byte
//    chunks of 1 KiB slabs, dot them against the matching slice of the query
//    in registers and reduce across the few lanes of one (key, group).
//  * index_score_f32_kernel   - fp32 inputs: plain fp32 FMA loops.
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kIdxWaves = 8;
constexpr int kIdxThreads = 64 * kIdxWaves;
constexpr int kQT = 64 * kIdxWaves;  // queries per work-group (each wave 2 x 32 columns)
constexpr int kKC = 16;   // key blocks per work-group

template <int DI, int BS>
struct IdxTile {
  static constexpr int CPR = DI / 8;                 // 16-byte chunks per key row
  static constexpr int CHUNKS = BS * CPR;            // chunks per key block
  static constexpr int CPT = (CHUNKS + kIdxThreads - 1) / kIdxThreads;  // chunks per thread
  static constexpr int STAGE = CHUNKS * 16;          // bytes per staged block
  static constexpr int RPB = 16 / CPR;               // rows sharing one 64-bank line
  static_assert(CHUNKS % kIdxThreads == 0 || CHUNKS < kIdxThreads, "uneven block split");
  // LDS position of 16-byte chunk q of key row r: chunks are XOR-swizzled so
  // the 32 rows read by one MFMA operand load hit distinct banks.
  __device__ static __forceinline__ int swz(int r, int q) { return r * CPR + (q ^ ((r / RPB) % CPR)); }
};

// One direct global-to-LDS load of 16 bytes per lane: lane l's bytes land at
// lds + 16 * l (`lds` is wave-uniform).  Kept out of the kernel body, where
// the host pass would reject the builtin and drop the kernel's launch stub.
__device__ __forceinline__ void dma16(const uint16_t *src, uint8_t *lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)lds, 16, 0, 0);
}

template <int DI, int BS>
__global__ __launch_bounds__(kIdxThreads) __attribute__((amdgpu_waves_per_eu(DI >= 128 ? 2 : 4, DI >= 128 ? 2 : 4))) void index_score_mfma_kernel(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    float *__restrict__ scores, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int G, int nb_max, int64_t total_q, int nqt, int nkcl) {
  using T = IdxTile<DI, BS>;
  constexpr int QT = kQT, KC = kKC, CPR = T::CPR, CPT = T::CPT;
  constexpr int KT = BS / 32;  // 32-key tiles per block
  constexpr int NK = DI / 16;  // MFMA steps over d_idx
  constexpr int RSTR = QT + 1; // result tile row stride (floats)
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[T::STAGE];
  __shared__ float res[KC * RSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  // Work-groups are dealt to the 8 XCDs round-robin (w runs on XCD w % 8).
  // Each XCD owns whole key chunks and runs the query tiles of one chunk back
  // to back, so the chunk's index keys are read from HBM once into that XCD's
  // L2 and reused by every query tile.  Chunks go to XCDs in snake order
  // (slot s of XCD x is chunk 8s + x for even s, 8s + 7 - x for odd s), which
  // balances the causal triangle's uneven chunks across XCDs.
  const int x = blockIdx.x & 7;
  int local = blockIdx.x >> 3;
  const int qt = nqt - 1 - local % nqt;
  local /= nqt;
  const int slot = local % nkcl;
  const int bg = local / nkcl;
  const int kc = 8 * slot + ((slot & 1) ? 7 - x : x);
  if (kc * KC >= nb_max) return;
  const int b = bg / G, g = bg - b * G;
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t t0 = (int64_t)qt * QT;
  if (t0 >= sq.lq) return;
  const int nq = (int)min<int64_t>(QT, sq.lq - t0);
  const int j0 = kc * KC;
  if (j0 >= nb_max) return;
  const int j1 = min(j0 + KC, nb_max);
  const int ncol = j1 - j0;
  const int64_t p_first = sq.base + t0, p_last = sq.base + t0 + nq - 1;
  const int64_t jmax = p_last < 0 ? -1 : p_last / BS;
  // blocks >= jmask may hold keys past some query's position
  const int jmask = p_first < 0 ? 0 : (int)(p_first / BS);
  const int jc_end = (int)min<int64_t>(j1, jmax + 1);
  const int nblk = max(0, jc_end - j0);
  float *out_rows = scores + ((int64_t)g * total_q + sq.q0 + t0) * nb_max + j0;

  if (nblk > 0) {
    // The tile's index queries as B operands (Q^T: d_idx x queries).
    bf16x8 qb[2][NK];
    int lim0[2];  // key limits relative to block j0: key s is causal iff s <= pos
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int qn = wave * 64 + s * 32 + col;
      const int64_t pos = sq.base + t0 + qn;
      lim0[s] = (int)min<int64_t>(max<int64_t>(pos - (int64_t)j0 * BS, -1), (int64_t)KC * BS);
      if (qn < nq) {
        const uint16_t *src = q_idx + ((sq.q0 + t0 + qn) * G + g) * (int64_t)DI + 8 * half;
#pragma unroll
        for (int c = 0; c < NK; ++c) qb[s][c] = as_bf16x8(ld16(src + 16 * c));
      } else {
#pragma unroll
        for (int c = 0; c < NK; ++c) qb[s][c] = zero_bf16x8();
      }
    }

    // Register staging (masked blocks only): thread tid moves chunks
    // tid + 512*i of a block; chunk P is key row P / CPR, 16-byte column
    // P % CPR, stored at its swizzled place.
    const int64_t kstride = (int64_t)G * DI;
    const uint16_t *kbase = k_idx + ((sq.kv0 + (int64_t)j0 * BS) * G + g) * (int64_t)DI;
    const int64_t rows_left = sq.lkv - (int64_t)j0 * BS;  // key rows of the chunk that exist
    auto fetch = [&](int it, u32x4 (&regs)[CPT]) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int P = tid + kIdxThreads * i;
        if (P >= T::CHUNKS) break;
        const int r = P / CPR, c = P % CPR;
        // rows past the sequence end are read from its last row (masked later)
        const int64_t row = min<int64_t>((int64_t)it * BS + r, rows_left - 1);
        regs[i] = ld16(kbase + row * kstride + 8 * c);
      }
    };
    auto store = [&](const u32x4 (&regs)[CPT], uint8_t *dst) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int P = tid + kIdxThreads * i;
        if (P >= T::CHUNKS) break;
        st16(dst + 16 * T::swz(P / CPR, P % CPR), regs[i]);
      }
    };

    // Direct loads into LDS (global_load_lds_dwordx4) for the unmasked
    // blocks: a block is NLD wave-loads of 64 16-byte slots, load L filling
    // slots [64L, 64L + 64) and wave w issuing loads w, w + 8, ...  Lane l of
    // load L fetches the chunk that the swizzle places in slot 64L + l.  All
    // rows of these blocks exist, so each lane steps one pointer per load by
    // a block per block.
    constexpr int NLD = T::CHUNKS / 64;
    constexpr int LPW = (NLD + kIdxWaves - 1) / kIdxWaves;  // loads per wave
    static_assert(T::CHUNKS % 64 == 0, "whole 64-slot loads");
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint16_t *kdma[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int S = min(64 * (wave_u + kIdxWaves * i) + lane, T::CHUNKS - 1);
      const int r = S / CPR;
      kdma[i] = kbase + r * kstride + 8 * ((S % CPR) ^ ((r / T::RPB) % CPR));
    }
    const int64_t kblock = (int64_t)BS * kstride;
    auto dma = [&](int it, uint8_t *dst) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int L = wave_u + kIdxWaves * i;
        if (NLD % kIdxWaves != 0 && L >= NLD) break;
        dma16(kdma[i] + it * kblock, dst + 1024 * L);
      }
    };

    // MFMAs of one key tile of the staged block `cur` (32 keys x 2 x 32 queries)
    auto mma = [&](const uint8_t *cur, int kt, f32x16 (&a)[2]) {
      const int r = kt * 32 + col;
      a[0] = f32x16{};
      a[1] = f32x16{};
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        const bf16x8 op = as_bf16x8(*reinterpret_cast<const u32x4 *>(
            cur + 16 * T::swz(r, 2 * c + half)));
        a[0] = mfma32x32x16(op, qb[0][c], a[0]);
        a[1] = mfma32x32x16(op, qb[1][c], a[1]);
      }
    };
    // Lanes l and l + 32 hold different keys of the same query column: after
    // the cross-half max, lane l stores query wave*64 + l (columns of half 0
    // from the low lanes, of half 1 from the high lanes).
    auto put = [&](int it, float m0, float m1) {
      res[it * RSTR + wave * 64 + lane] = halves_max_f(m0, m1);
    };

    // Blocks below jmask are causal for every query of the tile: a pipelined
    // loop without masking.  Block it sits in LDS stage `cur` while block
    // it+1 streams into `other`.  At the top of each step every wave waits
    // for its own direct loads (the only vector-memory operations in flight
    // here), then the barrier publishes the whole block to the work-group;
    // the work-group fence alone would not wait for loads that write LDS.
    // The two stages are separate LDS arrays, so the compiler can tell that
    // operand reads of `cur` need not wait for the loads into `other`.
    const int nfull = min(nblk, max(0, jmask - j0));
    auto step = [&](int it, const uint8_t *cur, uint8_t *other) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // block it in `cur`; every wave is done with `other`
      if (it + 1 < nfull) dma(it + 1, other);
      // Skewed schedule: the max over query half 0 of key tile kt runs while
      // the MFMAs of half 1 execute, and the max over half 1 while the MFMAs
      // of half 0 of tile kt+1 execute, so the block-max VALU work overlaps
      // the matrix pipe instead of following it.
      float m0 = neg_inf(), m1 = neg_inf();
      f32x16 a0, a1;
      auto mfma_half = [&](f32x16 &a, const u32x4 (&kf)[NK], int sq) {
        a = f32x16{};
#pragma unroll
        for (int c = 0; c < NK; ++c) a = mfma32x32x16(as_bf16x8(kf[c]), qb[sq][c], a);
      };
      auto max_into = [&](float &m, const f32x16 &a) {
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, a[e]);
      };
      // interleave: one MFMA, then two VALU ops (the 16-value max of the other
      // half is 8 v_max3), for the NK MFMAs just issued
      auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      };
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        u32x4 kf[NK];
        const int r = kt * 32 + col;
#pragma unroll
        for (int c = 0; c < NK; ++c)
          kf[c] = *reinterpret_cast<const u32x4 *>(cur + 16 * T::swz(r, 2 * c + half));
        mfma_half(a0, kf, 0);
        if (kt > 0) max_into(m1, a1);  // half 1 of tile kt-1
        interleave();
        mfma_half(a1, kf, 1);
        max_into(m0, a0);              // half 0 of tile kt
        interleave();
      }
      max_into(m1, a1);
      put(it, m0, m1);
    };
    if (nfull > 0) {
      dma(0, stage0);
      for (int it = 0; it < nfull; it += 2) {
        step(it, stage0, stage1);
        if (it + 1 < nfull) step(it + 1, stage1, stage0);
      }
    }

    // The tile's last blocks (its current blocks): causal mask, plain staging.
    for (int it = nfull; it < nblk; ++it) {
      u32x4 rr[CPT];
      fetch(it, rr);
      __syncthreads();  // every wave is done with stage 0
      store(rr, stage0);
      __syncthreads();
      const int l0 = lim0[0] - it * BS, l1 = lim0[1] - it * BS;
      float m0 = neg_inf(), m1 = neg_inf();
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x16 a[2];
        mma(stage0, kt, a);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
          m0 = fmaxf(m0, key > l0 ? neg_inf() : a[0][e]);
          m1 = fmaxf(m1, key > l1 ? neg_inf() : a[1][e]);
        }
      }
      put(it, m0, m1);
    }
  }
  // blocks of the chunk that no query of the tile reaches
  for (int i = tid; i < (ncol - nblk) * QT; i += kIdxThreads)
    res[(nblk + i / QT) * RSTR + (i % QT)] = neg_inf();
  __syncthreads();
  if (ncol == KC && nb_max % 4 == 0) {
    // full chunk: 4 consecutive blocks of one query row per 16-byte store
    // (rows start 16-byte aligned: nb_max and j0 are multiples of 4)
    constexpr int QPR = KC / 4;  // 16-byte pieces per query row
    for (int i = tid; i < nq * QPR; i += kIdxThreads) {
      const int r = i / QPR, c4 = 4 * (i % QPR);
      const float4 v = {res[c4 * RSTR + r], res[(c4 + 1) * RSTR + r], res[(c4 + 2) * RSTR + r],
                        res[(c4 + 3) * RSTR + r]};
      *reinterpret_cast<float4 *>(out_rows + (int64_t)r * nb_max + c4) = v;
    }
  } else {
    for (int i = tid; i < nq * ncol; i += kIdxThreads) {
      const int r = i / ncol, c = i - (i / ncol) * ncol;
      out_rows[(int64_t)r * nb_max + c] = res[c * RSTR + r];
    }
  }
}

// Sum over aligned groups of LPD lanes (4, 8 or 16) with DPP lane moves:
// swap neighbours, swap pairs, then fold the mirrored half of the 8-lane and
// 16-lane row.  Every lane of a group ends with the group's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int LPD>
__device__ __forceinline__ float lane_group_sum(float a) {
  a += dpp_mov<0xB1>(a);                       // quad_perm(1,0,3,2)
  a += dpp_mov<0x4E>(a);                       // quad_perm(2,3,0,1)
  if constexpr (LPD >= 8) a += dpp_mov<0x141>(a);   // row_half_mirror
  if constexpr (LPD >= 16) a += dpp_mov<0x140>(a);  // row_mirror
  return a;
}

// One work-group per key block.  Lane l reads 16-byte chunk l of each 1 KiB
// slab of the packed [key][group][d_idx] index-key rows (KPS keys share a
// slab), and wave w takes slabs w, w+4, ..., so the four waves stream 4 KiB of
// contiguous keys per step.  The block index is uniform, so the slab loop over
// a full block keeps eight loads per wave in flight; only a block cut by the
// causal end takes a predicated last slab.
template <int DI, int KPS>
__global__ __launch_bounds__(256) void index_score_decode_kernel(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    float *__restrict__ scores, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int G, int BS, int nb_max, int64_t total_q) {
  constexpr int LPD = DI / 8;  // lanes per (key, group) dot product
  __shared__ float wave_max[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int rowlen = 512 / KPS;  // G * DI elements per key
  const int b = blockIdx.y;
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int j = blockIdx.x;
  const int64_t row = sq.q0;
  const int64_t p = sq.base;  // the query's position: len_kv - 1
  const int e = lane * 8;
  const int key_in_slab = e / rowlen;
  const int g = (e % rowlen) / DI;
  const int dof = e % DI;
  const bool writer = wave == 0 && key_in_slab == 0 && dof == 0;
  float *dst = scores + ((int64_t)g * total_q + row) * nb_max + j;
  const int64_t s_begin = (int64_t)j * BS;
  // One branch for both exits: a sequence with no query row, and a block that
  // starts past the query (also p < 0: an empty cache).
  if (sq.lq <= 0 || s_begin > p) {
    if (sq.lq > 0 && writer) *dst = neg_inf();
    return;
  }
  const u32x4 qw = ld16(q_idx + (row * G + g) * (int64_t)DI + dof);
  float qf[8];
  auto dot = [&](const u32x4 w) {
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = fmaf(qf[2 * t], bf16_lo(w[t]), acc);
      acc = fmaf(qf[2 * t + 1], bf16_hi(w[t]), acc);
    }
    return lane_group_sum<LPD>(acc);
  };
  const int nkeys = (int)(min<int64_t>(s_begin + BS, p + 1) - s_begin);
  const int nfull = nkeys / KPS;  // slabs whose keys are all causal
  const int nslab = nfull + (nfull * KPS < nkeys ? 1 : 0);  // incl. a causally cut slab
  const uint16_t *blk = k_idx + (sq.kv0 + s_begin) * (int64_t)rowlen;
  const int in_row = e - key_in_slab * rowlen;  // this lane's offset within a key row
  // Wave w reads slabs w, w+4, ..., w+28 of a batch; rows past the block's
  // last causal key are clamped to it (those loads stay in bounds and their
  // values are never used).  The index-key cache is streamed once per step:
  // non-temporal loads.
  u32x4 w[8];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = min((i0 + 4 * u) * KPS + key_in_slab, nkeys - 1);
      w[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>(blk + (int64_t)r * rowlen + in_row));
    }
  };
  float mx = neg_inf();
  int i = wave;
  // The first batch is in flight before the query slice is waited for, and it
  // is used on every path, so it is not moved behind a branch.
  load_batch(i);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    qf[2 * t] = bf16_lo(qw[t]);
    qf[2 * t + 1] = bf16_hi(qw[t]);
  }
  while (i + 28 < nfull) {
#pragma unroll
    for (int u = 0; u < 8; ++u) mx = fmaxf(mx, dot(w[u]));
    i += 32;
    if (i < nslab) load_batch(i);
  }
  // Fewer than eight of this wave's slabs are left, all in w.
  if (i < nslab) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sl = i + 4 * u;
      const bool live = sl < nfull || (sl == nfull && nfull * KPS + key_in_slab < nkeys);
      const float acc = dot(w[u]);
      if (live) mx = fmaxf(mx, acc);
    }
  }
  for (int off = rowlen / 8; off < 64; off <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
  wave_max[wave][lane] = mx;
  __syncthreads();
  if (writer)
    *dst = fmaxf(fmaxf(wave_max[0][lane], wave_max[1][lane]),
                 fmaxf(wave_max[2][lane], wave_max[3][lane]));
}

__global__ __launch_bounds__(256) void index_score_f32_kernel(
    const float *__restrict__ q_idx, const float *__restrict__ k_idx, float *__restrict__ scores,
    const int64_t *__restrict__ cu_q, const int64_t *__restrict__ cu_kv, int num_seqs, int G,
    int DI, int BS, int nb_max, int64_t total_q) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int g = blockIdx.y;
  if (idx >= total_q * nb_max) return;
  const int64_t row = idx / nb_max;
  const int j = (int)(idx - row * nb_max);
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  float best = neg_inf();
  if (p >= 0 && (int64_t)j <= p / BS) {
    const float *q = q_idx + (row * G + g) * (int64_t)DI;
    const int64_t s_end = min<int64_t>((int64_t)j * BS + BS, p + 1);
    for (int64_t s = (int64_t)j * BS; s < s_end; ++s) {
      const float *k = k_idx + ((sq.kv0 + s) * G + g) * (int64_t)DI;
      float acc = 0.f;
      for (int c = 0; c < DI; ++c) acc = fmaf(q[c], k[c], acc);
      best = fmaxf(best, acc);
    }
  }
  scores[((int64_t)g * total_q + row) * nb_max + j] = best;
}

template <int DI, int BS>
hipError_t launch_mfma(const Dims &p, const uint16_t *q_idx, const uint16_t *k_idx, float *scores,
                       hipStream_t s) {
  const int nkc = (p.nb_max + kKC - 1) / kKC;   // key chunks
  const int nkcl = (nkc + 7) / 8;                // chunk slots per XCD
  const int nqt = (p.max_q_len + kQT - 1) / kQT; // query tiles
  const int64_t nwg = (int64_t)8 * nkcl * nqt * p.num_seqs * p.G;
  if (nwg > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((index_score_mfma_kernel<DI, BS>), dim3((unsigned)nwg), dim3(kIdxThreads), 0,
                     s, q_idx, k_idx, scores, p.cu_q, p.cu_kv, p.G, p.nb_max, p.total_q, nqt,
                     nkcl);
  profile_mark(s);
  return hipGetLastError();
}

template <int DI, int KPS>
hipError_t launch_decode(const Dims &p, const uint16_t *q_idx, const uint16_t *k_idx,
                         float *scores, hipStream_t s) {
  dim3 grid(p.nb_max, p.num_seqs);
  hipLaunchKernelGGL((index_score_decode_kernel<DI, KPS>), grid, dim3(256), 0, s, q_idx, k_idx,
                     scores, p.cu_q, p.cu_kv, p.G, p.B, p.nb_max, p.total_q);
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_score_bf16(const Dims &p, const uint16_t *q_idx, const uint16_t *k_idx,
                                   float *scores, hipStream_t s) {
  if (p.max_q_len <= 0 || p.nb_max <= 0) return hipSuccess;
#define MSA_IDX_CASE(DI_, BS_) \
  if (p.d_idx == DI_ && p.B == BS_) return launch_mfma<DI_, BS_>(p, q_idx, k_idx, scores, s);
  MSA_IDX_CASE(32, 64) MSA_IDX_CASE(32, 128) MSA_IDX_CASE(64, 64) MSA_IDX_CASE(64, 128)
  MSA_IDX_CASE(128, 64) MSA_IDX_CASE(128, 128)
#undef MSA_IDX_CASE
  return hipErrorInvalidValue;
}

bool decode_index_supported(const Dims &p) {
  const int rowlen = p.G * p.d_idx;
  return p.max_q_len == 1 && rowlen <= 512 && 512 % rowlen == 0;
}

hipError_t launch_index_score_decode_bf16(const Dims &p, const uint16_t *q_idx,
                                          const uint16_t *k_idx, float *scores, hipStream_t s) {
  if (p.nb_max <= 0) return hipSuccess;
  const int kps = 512 / (p.G * p.d_idx);
#define MSA_DEC_CASE(DI_, KPS_) \
  if (p.d_idx == DI_ && kps == KPS_) return launch_decode<DI_, KPS_>(p, q_idx, k_idx, scores, s);
  MSA_DEC_CASE(32, 1) MSA_DEC_CASE(32, 2) MSA_DEC_CASE(32, 4) MSA_DEC_CASE(32, 8)
  MSA_DEC_CASE(32, 16) MSA_DEC_CASE(64, 1) MSA_DEC_CASE(64, 2) MSA_DEC_CASE(64, 4)
  MSA_DEC_CASE(64, 8) MSA_DEC_CASE(128, 1) MSA_DEC_CASE(128, 2) MSA_DEC_CASE(128, 4)
#undef MSA_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_index_score_f32(const Dims &p, const float *q_idx, const float *k_idx,
                                  float *scores, hipStream_t s) {
  const int64_t n = p.total_q * p.nb_max;
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256), p.G);
  hipLaunchKernelGGL(index_score_f32_kernel, grid, dim3(256), 0, s, q_idx, k_idx, scores, p.cu_q,
                     p.cu_kv, p.num_seqs, p.G, p.d_idx, p.B, p.nb_max, p.total_q);
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace msa
