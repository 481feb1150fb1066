// Index Branch block scoring ("MiniMax Sparse Attention" page, Summary,
// paragraph 2): every key/value block is scored by max-pooling the
// token-level dot products of a query's index vector with the block's index
// keys.  scores[g, row, j] = max over causal keys s of block j of
// <q_idx[row, g], k_idx[s, g]>, and -inf where block j holds no causal key.
//
// Three kernels:
//  * index_score_mfma_kernel  - bf16 prefill.  A work-group owns 256 queries
//    x 32 key blocks of one (sequence, group).  The 256 index queries stay in
//    registers as MFMA B operands for the whole work-group; key blocks are
//    staged through LDS (register prefetch of the next block); each wave
//    computes S^T = K * Q^T tiles (keys x queries) with 32x32x16 bf16 MFMA so
//    a lane holds 16 keys of ONE query column and the block max is an in-lane
//    max chain plus one cross-half step.  Causal masking is applied only to
//    blocks that can hold keys past a query's position.
//  * index_score_decode_kernel - bf16, one query per sequence: a streaming
//    scan of the index-key cache (HBM-bound).  Lanes read consecutive 16-byte
//    chunks of 1 KiB slabs, dot them against the matching slice of the query
//    in registers and reduce across the few lanes of one (key, group).
//  * index_score_f32_kernel   - fp32 inputs: plain fp32 FMA loops.
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kQT = 256;  // queries per work-group (4 waves x 2 x 32 columns)
constexpr int kKC = 32;   // key blocks per work-group

template <int DI, int BS>
__global__ __launch_bounds__(256) void index_score_mfma_kernel(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    float *__restrict__ scores, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int G, int nb_max, int64_t total_q) {
  constexpr int QT = kQT, KC = kKC;
  constexpr int KT = BS / 32;        // 32-key tiles per block
  constexpr int NK = DI / 16;        // MFMA steps over d_idx
  constexpr int KROW = DI + 8;       // LDS row stride in bf16 (+16 B vs bank conflicts)
  constexpr int CPR = DI / 8;        // 16-byte chunks per key row
  constexpr int CPT = BS * CPR / 256;
  static_assert((BS * CPR) % 256 == 0, "a block must split evenly over 256 threads");
  constexpr int RSTR = QT + 1;       // LDS result row stride (floats)

  __shared__ __attribute__((aligned(16))) uint16_t ks[BS * KROW];
  __shared__ float res[KC * RSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int kc = blockIdx.x, qt = blockIdx.y, bg = blockIdx.z;
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
  const int jmask = p_first < 0 ? 0 : (int)(p_first / BS);
  const int jc_end = (int)min<int64_t>(j1, jmax + 1);
  float *out_rows = scores + ((int64_t)g * total_q + sq.q0 + t0) * nb_max + j0;

  if (jc_end <= j0) {  // no query of the tile reaches this chunk
    for (int i = tid; i < nq * ncol; i += 256) {
      const int r = i / ncol;
      out_rows[(int64_t)r * nb_max + (i - r * ncol)] = neg_inf();
    }
    return;
  }

  // The tile's index queries as B operands (Q^T: d_idx x queries).
  bf16x8 qb[2][NK];
  int64_t pos[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int qn = wave * 64 + s * 32 + (lane & 31);
    pos[s] = sq.base + t0 + qn;
    if (qn < nq) {
      const uint16_t *src = q_idx + ((sq.q0 + t0 + qn) * G + g) * (int64_t)DI + 8 * half;
#pragma unroll
      for (int c = 0; c < NK; ++c) qb[s][c] = as_bf16x8(ld16(src + 16 * c));
    } else {
#pragma unroll
      for (int c = 0; c < NK; ++c) qb[s][c] = zero_bf16x8();
    }
  }

  const int64_t kstride = (int64_t)G * DI;
  const uint16_t *kbase = k_idx + (sq.kv0 * G + g) * (int64_t)DI;
  u32x4 pre[CPT];
  auto fetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + 256 * i;
      const int r = ci / CPR, c = ci - (ci / CPR) * CPR;
      const int64_t s = (int64_t)j * BS + r;
      if (s < sq.lkv) pre[i] = ld16(kbase + s * kstride + 8 * c);
      else pre[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  fetch(j0);
  for (int j = j0; j < jc_end; ++j) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + 256 * i;
      const int r = ci / CPR, c = ci - (ci / CPR) * CPR;
      st16(ks + r * KROW + 8 * c, pre[i]);
    }
    __syncthreads();
    if (j + 1 < jc_end) fetch(j + 1);

    const bool need_mask = j >= jmask;
    float m0 = neg_inf(), m1 = neg_inf();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      f32x16 a0 = {}, a1 = {};
      const uint16_t *arow = ks + (kt * 32 + (lane & 31)) * KROW + 8 * half;
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(arow + 16 * c));
        a0 = mfma32x32x16(a, qb[0][c], a0);
        a1 = mfma32x32x16(a, qb[1][c], a1);
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t s = (int64_t)j * BS + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (s > pos[0]) a0[r] = neg_inf();
          if (s > pos[1]) a1[r] = neg_inf();
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        m0 = fmaxf(m0, a0[r]);
        m1 = fmaxf(m1, a1[r]);
      }
    }
    m0 = fmaxf(m0, shfl_xor_f(m0, 32));
    m1 = fmaxf(m1, shfl_xor_f(m1, 32));
    if (lane < 32) {
      res[(j - j0) * RSTR + wave * 64 + lane] = m0;
      res[(j - j0) * RSTR + wave * 64 + 32 + lane] = m1;
    }
  }
  for (int i = tid; i < (j1 - jc_end) * QT; i += 256)
    res[(jc_end - j0 + i / QT) * RSTR + (i % QT)] = neg_inf();
  __syncthreads();
  for (int i = tid; i < nq * ncol; i += 256) {
    const int r = i / ncol, c = i - (i / ncol) * ncol;
    out_rows[(int64_t)r * nb_max + c] = res[c * RSTR + r];
  }
}

// One wave per key block; lane l reads 16-byte chunk l of each 1 KiB slab of
// the packed [key][group][d_idx] index-key rows.  KPS keys share a slab.
template <int DI, int KPS>
__global__ __launch_bounds__(256) void index_score_decode_kernel(
    const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ k_idx,
    float *__restrict__ scores, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int G, int BS, int nb_max, int64_t total_q) {
  constexpr int LPD = DI / 8;  // lanes per (key, group) dot product
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  if (sq.lq <= 0) return;
  const int j = blockIdx.x * 4 + wave;
  if (j >= nb_max) return;
  const int64_t row = sq.q0;
  const int64_t p = sq.base;  // the query's position: len_kv - 1
  const int rowlen = G * DI;
  const int e = lane * 8;
  const int key_in_slab = e / rowlen;
  const int g = (e - key_in_slab * rowlen) / DI;
  const int dof = e - key_in_slab * rowlen - g * DI;
  const bool writer = key_in_slab == 0 && dof == 0;
  float *dst = scores + ((int64_t)g * total_q + row) * nb_max + j;
  const int64_t jmax = p < 0 ? -1 : p / BS;
  if ((int64_t)j > jmax) {
    if (writer) *dst = neg_inf();
    return;
  }
  float qf[8];
  {
    const u32x4 w = ld16(q_idx + (row * G + g) * (int64_t)DI + dof);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[2 * i] = bf16_lo(w[i]);
      qf[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  const int64_t s_begin = (int64_t)j * BS;
  const int nkeys = (int)(min<int64_t>(s_begin + BS, p + 1) - s_begin);
  const int nslab = (nkeys + KPS - 1) / KPS;
  const uint16_t *base = k_idx + (sq.kv0 + s_begin) * (int64_t)rowlen + e;
  float mx = neg_inf();
#pragma unroll 4
  for (int i = 0; i < nslab; ++i) {
    const int key = i * KPS + key_in_slab;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key < nkeys) w = ld16(base + (int64_t)i * 512);
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = fmaf(qf[2 * t], bf16_lo(w[t]), acc);
      acc = fmaf(qf[2 * t + 1], bf16_hi(w[t]), acc);
    }
#pragma unroll
    for (int off = 1; off < LPD; off <<= 1) acc += shfl_xor_f(acc, off);
    if (key < nkeys) mx = fmaxf(mx, acc);
  }
  for (int off = rowlen / 8; off < 64; off <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
  if (writer) *dst = mx;
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
  dim3 grid((p.nb_max + kKC - 1) / kKC, (p.max_q_len + kQT - 1) / kQT, p.num_seqs * p.G);
  hipLaunchKernelGGL((index_score_mfma_kernel<DI, BS>), grid, dim3(256), 0, s, q_idx, k_idx,
                     scores, p.cu_q, p.cu_kv, p.G, p.nb_max, p.total_q);
  return hipGetLastError();
}

template <int DI, int KPS>
hipError_t launch_decode(const Dims &p, const uint16_t *q_idx, const uint16_t *k_idx,
                         float *scores, hipStream_t s) {
  dim3 grid((p.nb_max + 3) / 4, p.num_seqs);
  hipLaunchKernelGGL((index_score_decode_kernel<DI, KPS>), grid, dim3(256), 0, s, q_idx, k_idx,
                     scores, p.cu_q, p.cu_kv, p.G, p.B, p.nb_max, p.total_q);
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
  return hipGetLastError();
}

}  // namespace msa
