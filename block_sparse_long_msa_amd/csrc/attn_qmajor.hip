// Main Branch attention, query-major ("MiniMax Sparse Attention" page,
// Summary, paragraph 2: exact softmax attention restricted to the kept
// blocks, for every query head of the group).
//
// One wave per (query row, KV group, split).  The hpg query heads of the
// group are the 16 columns of 16x16x32 bf16 MFMA tiles (heads >= hpg are
// zero columns), so every gathered K/V block is loaded once and shared by
// all heads of the group.  Per kept block:
//   S^T (keys x heads) = K (keys x d) . Q^T (d x heads)   K read straight
//                                                          from HBM as A
//   online softmax in fp32, log2 domain, per head column
//   O^T (dv x heads) += V^T (dv x keys) . P^T (keys x heads)
// V is staged through LDS transposed (dv-major) 32 keys at a time so the
// A operand of the second product is two 8-byte LDS reads per lane.  The
// P^T operand is built directly from the S^T accumulators: a lane's four
// keys of two adjacent 16-key tiles become its eight contraction elements,
// and V^T is read with the same key order.
//
// With n_split > 1 the kept-block list of a row is cut into splits (split-KV
// decoding); each split writes a normalised partial (O / l) and its LSE,
// and combine_splits_kernel merges them.
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

template <int D, int BS>
__global__ __launch_bounds__(64) void attn_qmajor_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ block_idx,
    uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part_o,
    float *__restrict__ part_lse, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int num_seqs, int H, int G, int K, int64_t total_q,
    float scale_log2, int n_split, int bps) {
  constexpr int NKT = BS / 16;  // 16-key S^T tiles per block
  constexpr int NDC = D / 32;   // MFMA steps over d in Q.K
  constexpr int NDT = D / 16;   // 16-row dv tiles of O^T
  constexpr int VROW = 36;      // LDS row stride (bf16) of the 32-key V^T chunk
  constexpr int OCT = D / 8;    // 16-byte octets per V row
  constexpr int TASKS = 8 * OCT;  // (key quad, dv octet) transposition tasks per chunk
  constexpr int TPL = TASKS / 64;  // tasks per lane
  static_assert(TASKS % 64 == 0, "whole tasks per lane");
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VROW];

  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t row = blockIdx.x;
  const int g = blockIdx.y;
  const int sp = blockIdx.z;
  const int hpg = H / G;
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  const int32_t *bidx = block_idx + ((int64_t)g * total_q + row) * K;
  const int slot0 = sp * bps, slot1 = min(K, slot0 + bps);
  const int64_t kvstride = (int64_t)G * D;

  bf16x8 qb[NDC];
  const bool head_ok = col < hpg;
  {
    const uint16_t *qrow = q + (row * H + g * hpg + (head_ok ? col : 0)) * (int64_t)D + 8 * grp;
#pragma unroll
    for (int c = 0; c < NDC; ++c) qb[c] = head_ok ? as_bf16x8(ld16(qrow + 32 * c)) : zero_bf16x8();
  }

  f32x4 o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = neg_inf(), l = 0.f;
  u32x4 wv[TPL][4];  // V rows of one 32-key chunk, in flight or being transposed

  for (int slot = slot0; slot < slot1; ++slot) {
    const int j = bidx[slot];
    if (j < 0) continue;
    const int64_t s0 = (int64_t)j * BS;
    if (p < s0) continue;  // not a causal block of this row (ignored)
    MSA_DCHECK(s0 < sq.lkv);
    const uint16_t *kblk = k + ((sq.kv0 + s0) * G + g) * (int64_t)D;
    const uint16_t *vblk = v + ((sq.kv0 + s0) * G + g) * (int64_t)D;

    // Keys past the sequence end read its last key instead (their scores are
    // masked below, and the V rows they stand for get weight 0), so every
    // load of the block is unconditional and they can all be in flight.
    const int nkey = (int)min<int64_t>(BS, sq.lkv - s0);
    auto load_v = [&](int ch) {
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const int task = lane + 64 * i, kq = task / OCT, o8 = task - (task / OCT) * OCT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = min(ch * 32 + 4 * kq + r, nkey - 1);
          wv[i][r] = ld16(vblk + key * kvstride + 8 * o8);
        }
      }
    };
    f32x4 st[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = min(kt * 16 + col, nkey - 1);
      const uint16_t *krow = kblk + key * kvstride + 8 * grp;
#pragma unroll
      for (int c = 0; c < NDC; ++c)
        st[kt] = mfma16x16x32(as_bf16x8(ld16(krow + 32 * c)), qb[c], st[kt]);
    }
    // V rows of the block's first 32-key chunk: (key quad, dv octet) tasks,
    // TPL per lane, loaded while the softmax runs
    load_v(0);
    float mb = neg_inf();
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t s = s0 + kt * 16 + 4 * grp + r;
        st[kt][r] = s > p ? neg_inf() : st[kt][r] * scale_log2;
        mb = fmaxf(mb, st[kt][r]);
      }
    }
    mb = xor32_max_f(xor16_max_f(mb));
    const float m_new = fmaxf(m, mb);  // finite: key s0 <= p is causal
    const float alpha = exp2f(m - m_new);
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st[kt][r] = exp2f(st[kt][r] - m_new);
        ps += st[kt][r];
      }
    }
    ps = xor32_sum_f(xor16_sum_f(ps));
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[t] *= alpha;

#pragma unroll
    for (int ch = 0; ch < BS / 32; ++ch) {
      __syncthreads();  // the previous chunk's V^T reads are done
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const int task = lane + 64 * i, kq = task / OCT, o8 = task - (task / OCT) * OCT;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          const uint32_t k0 = (wv[i][0][e >> 1] >> sh) & 0xffffu, k1 = (wv[i][1][e >> 1] >> sh) & 0xffffu;
          const uint32_t k2 = (wv[i][2][e >> 1] >> sh) & 0xffffu, k3 = (wv[i][3][e >> 1] >> sh) & 0xffffu;
          u32x2 pk = {k0 | (k1 << 16), k2 | (k3 << 16)};
          *reinterpret_cast<u32x2 *>(vt + (8 * o8 + e) * VROW + 4 * kq) = pk;
        }
      }
      // the next chunk's V rows load while this chunk's products run
      if (ch + 1 < BS / 32) load_v(ch + 1);
      __syncthreads();
      const f32x4 &p0 = st[2 * ch], &p1 = st[2 * ch + 1];
      u32x4 pw = {pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]),
                  pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3])};
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const uint16_t *vr = vt + (16 * t + col) * VROW + 4 * grp;
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 16);
        u32x4 aw = {lo[0], lo[1], hi[0], hi[1]};
        o[t] = mfma16x16x32(as_bf16x8(aw), pb, o[t]);
      }
    }
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float row_lse = l > 0.f ? (m + log2f(l)) * kLn2 : neg_inf();
  if (!head_ok) return;
  const int h = g * hpg + col;
  if (n_split == 1) {
    uint16_t *orow = out + (row * H + h) * (int64_t)D + 4 * grp;
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      u32x2 pk = {pack_bf16x2(o[t][0] * inv, o[t][1] * inv), pack_bf16x2(o[t][2] * inv, o[t][3] * inv)};
      *reinterpret_cast<u32x2 *>(orow + 16 * t) = pk;
    }
    if (lse != nullptr && grp == 0) lse[row * H + h] = row_lse;
  } else {
    float *prow = part_o + (((int64_t)sp * total_q + row) * H + h) * D + 4 * grp;
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      f32x4 val = o[t] * inv;
      *reinterpret_cast<f32x4 *>(prow + 16 * t) = val;
    }
    if (grp == 0) part_lse[((int64_t)sp * total_q + row) * H + h] = row_lse;
  }
}

// fp32 inputs: one wave per (query row, head, split); lanes take keys for
// the logits and value columns for the output; fp32 FMA throughout.
template <int D>
__global__ __launch_bounds__(64) void attn_qmajor_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const int32_t *__restrict__ block_idx, float *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ part_o, float *__restrict__ part_lse, const int64_t *__restrict__ cu_q,
    const int64_t *__restrict__ cu_kv, int num_seqs, int H, int G, int BS, int K,
    int64_t total_q, float scale, int n_split, int bps) {
  constexpr int DPL = D / 64;  // output columns per lane
  __shared__ float qs[D];
  __shared__ float pw[128];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y, sp = blockIdx.z;
  const int g = h / (H / G);
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t p = sq.base + (row - sq.q0);
  const int32_t *bidx = block_idx + ((int64_t)g * total_q + row) * K;
  const int slot0 = sp * bps, slot1 = min(K, slot0 + bps);
  const int64_t kvstride = (int64_t)G * D;
  for (int c = lane; c < D; c += 64) qs[c] = q[(row * H + h) * (int64_t)D + c];
  __syncthreads();
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float m = neg_inf(), l = 0.f;
  for (int slot = slot0; slot < slot1; ++slot) {
    const int j = bidx[slot];
    if (j < 0) continue;
    const int64_t s0 = (int64_t)j * BS;
    if (p < s0) continue;
    MSA_DCHECK(s0 < sq.lkv);
    const float *kb = k + ((sq.kv0 + s0) * G + g) * (int64_t)D;
    const float *vb = v + ((sq.kv0 + s0) * G + g) * (int64_t)D;
    const int nk = (int)min<int64_t>(BS, p + 1 - s0);  // causal keys of this block
    float z[2];
    float mb = neg_inf();
    for (int i = 0; i < 2; ++i) {
      const int key = lane + 64 * i;
      z[i] = neg_inf();
      if (key < nk) {
        const float *kr = kb + key * kvstride;
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc = fmaf(qs[c], kr[c], acc);
        z[i] = acc * scale;
      }
      mb = fmaxf(mb, z[i]);
    }
    for (int off = 32; off >= 1; off >>= 1) mb = fmaxf(mb, shfl_xor_f(mb, off));
    const float m_new = fmaxf(m, mb);
    const float alpha = expf(m - m_new);
    float ps = 0.f;
    for (int i = 0; i < 2; ++i) {
      const float e = z[i] == neg_inf() ? 0.f : expf(z[i] - m_new);
      ps += e;
      if (lane + 64 * i < 128) pw[lane + 64 * i] = e;
    }
    for (int off = 32; off >= 1; off >>= 1) ps += shfl_xor_f(ps, off);
    l = l * alpha + ps;
    m = m_new;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      float acc = o[i] * alpha;
      for (int t = 0; t < nk; ++t) acc = fmaf(pw[t], vb[t * kvstride + lane + 64 * i], acc);
      o[i] = acc;
    }
    __syncthreads();
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float row_lse = l > 0.f ? m + logf(l) : neg_inf();
  if (n_split == 1) {
#pragma unroll
    for (int i = 0; i < DPL; ++i) out[(row * H + h) * (int64_t)D + lane + 64 * i] = o[i] * inv;
    if (lse != nullptr && lane == 0) lse[row * H + h] = row_lse;
  } else {
    float *prow = part_o + (((int64_t)sp * total_q + row) * H + h) * D;
#pragma unroll
    for (int i = 0; i < DPL; ++i) prow[lane + 64 * i] = o[i] * inv;
    if (lane == 0) part_lse[((int64_t)sp * total_q + row) * H + h] = row_lse;
  }
}

// Merge of split partials: one wave per (row, head), lanes over d.
__global__ __launch_bounds__(256) void combine_splits_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse, void *__restrict__ out,
    int out_bf16, float *__restrict__ lse, int64_t total_q, int H, int D, int n_split) {
  const int lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row * H + h
  if (rh >= total_q * H) return;
  const int64_t plane = total_q * H;
  float M = neg_inf();
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_lse[s * plane + rh]);
  float acc[2] = {0.f, 0.f};
  float W = 0.f;
  if (M != neg_inf()) {
    for (int s = 0; s < n_split; ++s) {
      const float ls = part_lse[s * plane + rh];
      if (ls == neg_inf()) continue;
      const float w = expf(ls - M);
      W += w;
      const float *po = part_o + (s * plane + rh) * D;
      for (int i = 0; i < 2; ++i)
        if (lane + 64 * i < D) acc[i] = fmaf(w, po[lane + 64 * i], acc[i]);
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  for (int i = 0; i < 2; ++i) {
    const int c = lane + 64 * i;
    if (c >= D) continue;
    const float val = acc[i] * inv;
    if (out_bf16) reinterpret_cast<uint16_t *>(out)[rh * D + c] = (uint16_t)f32_to_bf16_bits(val);
    else reinterpret_cast<float *>(out)[rh * D + c] = val;
  }
  if (lse != nullptr && lane == 0) lse[rh] = W > 0.f ? M + logf(W) : neg_inf();
}

}  // namespace

MSA_DEBUG_COUNTER(attn_qmajor)

hipError_t launch_attn_qmajor_bf16(const Dims &p, const uint16_t *q, const uint16_t *k,
                                   const uint16_t *v, const int32_t *block_idx, uint16_t *out,
                                   float *lse, int n_split, float *part_o, float *part_lse,
                                   hipStream_t s) {
  if (p.total_q <= 0) return hipSuccess;
  const int bps = (p.top_k + n_split - 1) / n_split;
  dim3 grid((unsigned)p.total_q, p.G, n_split);
  const float sl2 = p.scale * kLog2e;
#define MSA_QM_CASE(D_, BS_)                                                                  \
  if (p.d == D_ && p.B == BS_) {                                                              \
    hipLaunchKernelGGL((attn_qmajor_bf16_kernel<D_, BS_>), grid, dim3(64), 0, s, q, k, v,     \
                       block_idx, out, lse, part_o, part_lse, p.cu_q, p.cu_kv, p.num_seqs,   \
                       p.H, p.G, p.top_k, p.total_q, sl2, n_split, bps);                     \
    profile_mark(s);                                                                          \
    return hipGetLastError();                                                                 \
  }
  MSA_QM_CASE(64, 64) MSA_QM_CASE(64, 128) MSA_QM_CASE(128, 64) MSA_QM_CASE(128, 128)
#undef MSA_QM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_qmajor_f32(const Dims &p, const float *q, const float *k, const float *v,
                                  const int32_t *block_idx, float *out, float *lse, int n_split,
                                  float *part_o, float *part_lse, hipStream_t s) {
  if (p.total_q <= 0) return hipSuccess;
  const int bps = (p.top_k + n_split - 1) / n_split;
  dim3 grid((unsigned)p.total_q, p.H, n_split);
  if (p.d == 64) {
    hipLaunchKernelGGL((attn_qmajor_f32_kernel<64>), grid, dim3(64), 0, s, q, k, v, block_idx,
                       out, lse, part_o, part_lse, p.cu_q, p.cu_kv, p.num_seqs, p.H, p.G, p.B,
                       p.top_k, p.total_q, p.scale, n_split, bps);
    profile_mark(s);
  } else if (p.d == 128) {
    hipLaunchKernelGGL((attn_qmajor_f32_kernel<128>), grid, dim3(64), 0, s, q, k, v, block_idx,
                       out, lse, part_o, part_lse, p.cu_q, p.cu_kv, p.num_seqs, p.H, p.G, p.B,
                       p.top_k, p.total_q, p.scale, n_split, bps);
    profile_mark(s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine_splits(const Dims &p, int n_split, const float *part_o,
                                 const float *part_lse, void *out, bool out_bf16, float *lse,
                                 hipStream_t s) {
  const int64_t n = p.total_q * p.H;
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 3) / 4));
  hipLaunchKernelGGL(combine_splits_kernel, grid, dim3(256), 0, s, part_o, part_lse, out,
                     out_bf16 ? 1 : 0, lse, p.total_q, p.H, p.d, n_split);
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace msa
