// Device-side helpers shared by the MSA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// bf16 <-> fp32.  bf16 is the top half of an fp32, so widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 narrowing with the hardware converter (v_cvt_pk_bf16_f32:
// round to nearest even, NaN stays NaN).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) {
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return as_bf16x8(z);
}

// LDS pointer type of the direct global-to-LDS load builtin.
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte loads (pointer must be 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, const u32x4 &v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

// MFMA wrappers.  Operand layouts (wave64):
//  32x32x16: A[i][k] in lane i + 32*(k/8), element k%8; B[k][j] in lane j + 32*(k/8);
//            C[i][j] in lane j + 32*((i/4)%2), register 4*(i/8) + i%4.
//  16x16x32: A[i][k] in lane i + 16*(k/8), element k%8; B[k][j] in lane j + 16*(k/8);
//            C[i][j] in lane j + 16*(i/4), register i%4.
// Only the row/column placement matters for correctness: the contraction
// index is summed, so any bijection of k used identically by A and B works.
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Cross-lane helpers (wave64).
__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
// max / sum of v over lanes l and l ^ 32, in every lane, with one
// v_permlane32_swap (a VALU lane swap between the wave's halves) instead of an
// LDS round trip.  Swapping v with itself leaves v[l] in one result and
// v[l ^ 32] in the other, whichever way the swap runs, so only the
// commutative combine of the two is used.
__device__ __forceinline__ float xor32_max_f(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum_f(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same over lanes l and l ^ 16 with v_permlane16_swap, which exchanges
// the odd 16-lane rows of one operand with the even rows of the other:
// swapping v with itself leaves each lane v[l] and v[l ^ 16].
__device__ __forceinline__ float xor16_max_f(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum_f(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// For two values per lane whose halves hold different parts of one column
// (lanes l and l + 32 share column l % 32): lane l < 32 gets the max of a over
// lanes l and l + 32, lane l >= 32 the max of b over lanes l - 32 and l.  One
// v_permlane32_swap exchanges the upper 32 lanes of a with the lower 32
// lanes of b; each lane then holds both of its pair's values.
__device__ __forceinline__ float halves_max_f(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
// DPP lane move within 16-lane rows (CTRL: 0xB1 swaps neighbours, 0x4E swaps
// pairs, 0x141 mirrors each 8-lane half row, 0x140 mirrors the row).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// Wave-uniform maximum / minimum of one value per lane: DPP steps reduce each
// 16-lane row, then the four row results are read into scalar registers.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  m = max(m, dpp_u32<0xB1>(m));
  m = max(m, dpp_u32<0x4E>(m));
  m = max(m, dpp_u32<0x141>(m));
  m = max(m, dpp_u32<0x140>(m));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t m) {
  m = min(m, dpp_u32<0xB1>(m));
  m = min(m, dpp_u32<0x4E>(m));
  m = min(m, dpp_u32<0x141>(m));
  m = min(m, dpp_u32<0x140>(m));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
}
// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int mbcnt64(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Per-sequence geometry.  Queries are the last len_q tokens of the sequence,
// so local query i sits at position base + i with base = len_kv - len_q.
struct SeqGeom {
  int64_t q0, lq, kv0, lkv, base;
};
__device__ __forceinline__ SeqGeom seq_geom(const int64_t *cu_q, const int64_t *cu_kv, int b) {
  SeqGeom s;
  s.q0 = cu_q[b];
  s.lq = cu_q[b + 1] - s.q0;
  s.kv0 = cu_kv[b];
  s.lkv = cu_kv[b + 1] - s.kv0;
  s.base = s.lkv - s.lq;
  return s;
}
// Sequence holding packed query row `row` (binary search over cu_q).
__device__ __forceinline__ int find_seq(const int64_t *cu_q, int num_seqs, int64_t row) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Debug builds (-DMSA_DEBUG, libmsa_debug.so): MSA_DCHECK(cond) evaluates a
// bounds condition of a gather in every active lane, and the wave's first
// active lane adds the number of lanes that checked and the number that
// failed to two device counters of the source file (internal linkage, one
// pair per file), so a broken index is reported by
// msa_debug_bounds_violations() rather than trapping.  The access itself is
// left as it is.  Release builds compile the checks away.
#ifdef MSA_DEBUG
namespace {
__device__ unsigned long long g_debug_checks;
__device__ unsigned long long g_debug_violations;
__device__ __forceinline__ void debug_check(bool ok) {
  const uint64_t act = __builtin_amdgcn_read_exec();
  const uint64_t bad = ballot64(!ok);
  if (mbcnt64(act) == 0) {  // first active lane
    atomicAdd(&g_debug_checks, (unsigned long long)__popcll(act));
    if (bad != 0) atomicAdd(&g_debug_violations, (unsigned long long)__popcll(bad));
  }
}
}  // namespace
#define MSA_DCHECK(cond) ::msa::debug_check(static_cast<bool>(cond))
// Host accessor of a file's counters (read, then optionally clear); false if
// the device could not be read.
#define MSA_DEBUG_COUNTER(name)                                                           \
  bool debug_counters_##name(uint64_t *checks, uint64_t *violations, bool reset) {        \
    unsigned long long c = 0, v = 0, z = 0;                                               \
    if (hipMemcpyFromSymbol(&c, HIP_SYMBOL(g_debug_checks), sizeof(c)) != hipSuccess ||   \
        hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_violations), sizeof(v)) != hipSuccess) \
      return false;                                                                       \
    if (reset && (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_checks), &z, sizeof(z)) != hipSuccess || \
                  hipMemcpyToSymbol(HIP_SYMBOL(g_debug_violations), &z, sizeof(z)) != hipSuccess)) \
      return false;                                                                       \
    *checks += c;                                                                         \
    *violations += v;                                                                     \
    return true;                                                                          \
  }
#else
#define MSA_DCHECK(cond) \
  do {                   \
  } while (0)
#define MSA_DEBUG_COUNTER(name)
#endif

}  // namespace msa
