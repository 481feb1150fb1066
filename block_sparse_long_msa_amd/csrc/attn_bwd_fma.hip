// Backward of the Main Branch ("MiniMax Sparse Attention" page, Summary,
// paragraph 2: exact softmax attention restricted to the keys of the kept
// blocks) with plain fp32 FMA, for every shape and dtype the forward takes:
// fp32 inputs, head dim 64, block size 64, any heads per group.  The same
// quantities as the MFMA path (attn_bwd.hip), in fp32 throughout:
//   D = <dO, O>,  P_s = exp(scale <q, k_s> - lse),  dS_s = P_s (<dO, v_s> - D)
//   dq = scale sum_s dS_s k_s (slots in order, keys ascending)
//   dk_s = scale sum dS_s q, dv_s = sum P_s dO over the (row, slot) entries
//          that keep s's block, in (row, slot) order, heads ascending
// Deterministic, no floating-point atomics.
//   fb_dsum   D per (row, head), one wave each
//   bk_*      bucket lists (buckets.hpp)
//   fb_dq     one wave per (row, head), lanes over channels
//   fb_dkv    one wave per (group, key), lanes over channels, walking the
//             list of the key's block
#include <algorithm>

#include "buckets.hpp"
#include "launch.hpp"
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kMaxCpl = 2;  // channels per lane (head dim <= 128)

struct FbWs {
  int32_t *cnt, *base, *lists, *ibase, *pbase;
  float *dsum;  // [total_q][H]
  int64_t ntiles, nbk_g, nent_g, tile;
  size_t total_bytes;
};

size_t fb_align(size_t x) { return (x + 255) & ~(size_t)255; }

FbWs fb_carve(const Dims &p, void *base) {
  FbWs w;
  w.nent_g = p.total_q * (int64_t)p.top_k;
  w.nbk_g = (int64_t)p.num_seqs * p.nb_max;
  w.tile = bucket_tile(w.nent_g, w.nbk_g);
  w.ntiles = (w.nent_g + w.tile - 1) / w.tile;
  size_t off = 0;
  char *c = static_cast<char *>(base);
  auto take = [&](size_t bytes) {
    char *r = c == nullptr ? nullptr : c + off;
    off += fb_align(bytes);
    return r;
  };
  w.cnt = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)p.G * w.ntiles * w.nbk_g));
  w.base = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  w.lists = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)p.G * w.nent_g));
  w.ibase = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  w.pbase = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * ((size_t)p.G * w.nbk_g + 1)));
  w.dsum = reinterpret_cast<float *>(take(sizeof(float) * (size_t)p.total_q * p.H));
  w.total_bytes = off;
  return w;
}

__device__ __forceinline__ float ld_f32(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float ld_f32(const float *p) { return *p; }

// Sum over the 64 lanes of a wave, the same fixed tree in every lane.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += shfl_xor_f(x, m);
  return x;
}

// lanes hold channels lane + 64 u, u < cpl (cpl = d / 64)
template <typename T>
__device__ __forceinline__ void load_row(const T *p, int cpl, int lane, float (&x)[kMaxCpl]) {
#pragma unroll
  for (int u = 0; u < kMaxCpl; ++u) x[u] = u < cpl ? ld_f32(p + lane + 64 * u) : 0.f;
}
__device__ __forceinline__ float dot_lanes(const float (&a)[kMaxCpl], const float (&b)[kMaxCpl]) {
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxCpl; ++u) s = fmaf(a[u], b[u], s);
  return wave_sum(s);
}

template <typename T>
__global__ __launch_bounds__(256) void fb_dsum_kernel(const T *__restrict__ out,
                                                      const T *__restrict__ dout,
                                                      float *__restrict__ dsum, int64_t nrows,
                                                      int d) {
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= nrows) return;
  const int lane = threadIdx.x & 63, cpl = d / 64;
  float o[kMaxCpl], g[kMaxCpl];
  load_row(out + rh * d, cpl, lane, o);
  load_row(dout + rh * d, cpl, lane, g);
  const float s = dot_lanes(o, g);
  if (lane == 0) dsum[rh] = s;
}

// One wave per (row, head).
template <typename T>
__global__ __launch_bounds__(256) void fb_dq_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const int32_t *__restrict__ block_idx, const float *__restrict__ lse,
    const T *__restrict__ dout, const float *__restrict__ dsum, float *__restrict__ dq,
    const int64_t *__restrict__ cu_q, const int64_t *__restrict__ cu_kv, int num_seqs, int H,
    int G, int d, int BS, int K, int64_t total_q, int nb_max, float scale) {
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= total_q * H) return;
  const int lane = threadIdx.x & 63, cpl = d / 64;
  const int64_t row = rh / H;
  const int h = (int)(rh - row * H), g = h / (H / G);
  const int b = find_seq(cu_q, num_seqs, row);
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t pos = sq.base + (row - sq.q0);
  float qr[kMaxCpl], gr[kMaxCpl], acc[kMaxCpl] = {};
  load_row(q + rh * d, cpl, lane, qr);
  load_row(dout + rh * d, cpl, lane, gr);
  const float l = lse[rh], D = dsum[rh];
  const int32_t *bi = block_idx + ((int64_t)g * total_q + row) * K;
  for (int i = 0; i < K; ++i) {
    const int j = bi[i];
    if (j < 0 || j >= nb_max || pos < 0 || (int64_t)j * BS > pos) continue;
    const int64_t s1 = min<int64_t>((int64_t)j * BS + BS - 1, pos);
    for (int64_t s = (int64_t)j * BS; s <= s1; ++s) {
      const int64_t kr = ((sq.kv0 + s) * G + g) * (int64_t)d;
      float kx[kMaxCpl], vx[kMaxCpl];
      load_row(k + kr, cpl, lane, kx);
      load_row(v + kr, cpl, lane, vx);
      const float p = expf(scale * dot_lanes(qr, kx) - l);
      const float ds = p * (dot_lanes(gr, vx) - D);
#pragma unroll
      for (int u = 0; u < kMaxCpl; ++u) acc[u] = fmaf(ds, kx[u], acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kMaxCpl; ++u)
    if (u < cpl) dq[rh * d + lane + 64 * u] = scale * acc[u];
}

// One wave per (group, key): the entries of the key's block list, in order.
template <typename T>
__global__ __launch_bounds__(256) void fb_dkv_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ lse, const T *__restrict__ dout, const float *__restrict__ dsum,
    const int32_t *__restrict__ base, const int32_t *__restrict__ lists, float *__restrict__ dk,
    float *__restrict__ dv, const int64_t *__restrict__ cu_q, const int64_t *__restrict__ cu_kv,
    int num_seqs, int H, int G, int d, int BS, int K, int64_t total_kv, int nb_max, float scale) {
  const int64_t gk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // key row * G + g
  if (gk >= total_kv * G) return;
  const int lane = threadIdx.x & 63, cpl = d / 64, hpg = H / G;
  const int64_t key = gk / G;
  const int g = (int)(gk - key * G);
  // the key's sequence (binary search over cu_kv) and block
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_kv[mid] <= key) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const SeqGeom sq = seq_geom(cu_q, cu_kv, b);
  const int64_t s = key - sq.kv0;
  const int j = (int)(s / BS);
  const int64_t nbk_g = (int64_t)num_seqs * nb_max;
  const int64_t gb = (int64_t)g * nbk_g + (int64_t)b * nb_max + j;
  float kx[kMaxCpl], vx[kMaxCpl], ak[kMaxCpl] = {}, av[kMaxCpl] = {};
  load_row(k + gk * d, cpl, lane, kx);
  load_row(v + gk * d, cpl, lane, vx);
  for (int32_t x = base[gb]; x < base[gb + 1]; ++x) {
    const int64_t row = lists[x] / K;
    if (s > sq.base + (row - sq.q0)) continue;  // past the row's position (current block)
    for (int hh = 0; hh < hpg; ++hh) {
      const int64_t rh = row * H + g * hpg + hh;
      float qr[kMaxCpl], gr[kMaxCpl];
      load_row(q + rh * d, cpl, lane, qr);
      load_row(dout + rh * d, cpl, lane, gr);
      const float p = expf(scale * dot_lanes(qr, kx) - lse[rh]);
      const float ds = p * (dot_lanes(gr, vx) - dsum[rh]);
#pragma unroll
      for (int u = 0; u < kMaxCpl; ++u) {
        av[u] = fmaf(p, gr[u], av[u]);
        ak[u] = fmaf(ds, qr[u], ak[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kMaxCpl; ++u)
    if (u < cpl) {
      dv[gk * d + lane + 64 * u] = av[u];
      dk[gk * d + lane + 64 * u] = scale * ak[u];
    }
}

__global__ __launch_bounds__(256) void fb_zero_kernel(float *__restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    x[i] = 0.f;
}

void fb_zero(float *x, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  const unsigned zg = (unsigned)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(fb_zero_kernel, dim3(zg), dim3(256), 0, s, x, n);
}

template <typename T>
hipError_t launch_fb(const Dims &p, const T *q, const T *k, const T *v, const int32_t *block_idx,
                     const T *out, const float *lse, const T *dout, float *dq, float *dk,
                     float *dv, void *workspace, hipStream_t s) {
  FbWs w = fb_carve(p, workspace);
  if (p.total_q == 0 || p.total_kv == 0) {  // nothing kept: all gradients are 0
    fb_zero(dk, p.total_kv * p.G * (int64_t)p.d, s);
    fb_zero(dv, p.total_kv * p.G * (int64_t)p.d, s);
    fb_zero(dq, p.total_q * p.H * (int64_t)p.d, s);
    profile_mark(s);
    return hipGetLastError();
  }
  const int64_t nrows = p.total_q * p.H;
  hipLaunchKernelGGL((fb_dsum_kernel<T>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, s, out,
                     dout, w.dsum, nrows, p.d);
  profile_mark(s);
  const size_t hist_bytes = sizeof(int32_t) * (size_t)w.nbk_g;
  hipLaunchKernelGGL(bk_count_kernel, dim3((unsigned)w.ntiles, p.G), dim3(256), hist_bytes, s,
                     block_idx, p.cu_q, p.cu_kv, w.cnt, nullptr, p.num_seqs, p.top_k, p.total_q,
                     (int64_t)0, w.nent_g, p.nb_max, p.B, w.ntiles, w.nbk_g, w.tile);
  const int64_t ncol = (int64_t)p.G * w.nbk_g;
  hipLaunchKernelGGL(bk_colscan_kernel, dim3((unsigned)((ncol + 255) / 256)), dim3(256), 0, s,
                     w.cnt, w.base, w.ibase, w.pbase, p.G, w.ntiles, w.nbk_g, 1 << 16);
  hipLaunchKernelGGL(bk_basescan_kernel, dim3(1), dim3(1024), 0, s, w.base, ncol);
  hipLaunchKernelGGL(bk_scatter_kernel, dim3((unsigned)w.ntiles, p.G), dim3(64), hist_bytes, s,
                     block_idx, p.cu_q, p.cu_kv, w.cnt, w.base, w.lists, p.num_seqs, p.top_k,
                     p.total_q, (int64_t)0, w.nent_g, p.nb_max, p.B, w.ntiles, w.nbk_g, w.tile);
  profile_mark(s);
  hipLaunchKernelGGL((fb_dq_kernel<T>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, s, q, k,
                     v, block_idx, lse, dout, w.dsum, dq, p.cu_q, p.cu_kv, p.num_seqs, p.H, p.G,
                     p.d, p.B, p.top_k, p.total_q, p.nb_max, p.scale);
  profile_mark(s);
  const int64_t nkg = p.total_kv * p.G;
  hipLaunchKernelGGL((fb_dkv_kernel<T>), dim3((unsigned)((nkg + 3) / 4)), dim3(256), 0, s, q, k,
                     v, lse, dout, w.dsum, w.base, w.lists, dk, dv, p.cu_q, p.cu_kv, p.num_seqs,
                     p.H, p.G, p.d, p.B, p.top_k, p.total_kv, p.nb_max, p.scale);
  profile_mark(s);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_fma_workspace_bytes(const Dims &p) {
  return p.total_q > 0 ? fb_carve(p, nullptr).total_bytes : 0;
}

hipError_t launch_attn_bwd_fma(const Dims &p, bool bf16, const void *q, const void *k,
                               const void *v, const int32_t *block_idx, const void *out,
                               const float *lse, const void *dout, float *dq, float *dk,
                               float *dv, void *workspace, hipStream_t s) {
  if (bf16)
    return launch_fb(p, static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                     static_cast<const uint16_t *>(v), block_idx,
                     static_cast<const uint16_t *>(out), lse,
                     static_cast<const uint16_t *>(dout), dq, dk, dv, workspace, s);
  return launch_fb(p, static_cast<const float *>(q), static_cast<const float *>(k),
                   static_cast<const float *>(v), block_idx, static_cast<const float *>(out), lse,
                   static_cast<const float *>(dout), dq, dk, dv, workspace, s);
}

}  // namespace msa
