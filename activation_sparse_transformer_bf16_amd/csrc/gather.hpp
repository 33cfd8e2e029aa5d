// Pieces shared by the gather kernels (sparse forward and backward) and the
// format conversions: row lookup in an ascending list, XCD
// placement of weight groups / column slices, raw buffer loads with a
// wave-uniform row offset, 16-byte dot products and joint wave reductions.
#pragma once

#include "common.hpp"

namespace twell {

// Position of row t in the ascending list rows[0..n), or -1.
__device__ __forceinline__ int find_row(const int *__restrict__ rows, int n, int t) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rows[mid] < t)
      lo = mid + 1;
    else
      hi = mid;
  }
  return (lo < n && rows[lo] == t) ? lo : -1;
}

constexpr int SP_THREADS = 256;
constexpr int SP_WAVES = SP_THREADS / 64;

// Block -> (group, token block).  With 8 or more groups, group g runs on XCD
// g % 8: groups are taken 8 at a time (a phase), the group count rounded up to
// a multiple of 8 (blocks of a missing group return at once), so that each
// XCD's L2 holds one group's weights per phase.  With fewer groups, group
// bid % n_groups (XCD x serves group x % n_groups).
__host__ __device__ constexpr int padded_groups(int n_groups) {
  return n_groups >= 8 ? (n_groups + 7) / 8 * 8 : n_groups;
}
__device__ __forceinline__ void group_coords(int bid, int n_groups, int n_tb, int &g, int &tb) {
  if (n_groups >= 8) {
    const int q = bid / 8;
    g = bid % 8 + 8 * (q / n_tb);
    tb = q % n_tb;
  } else {
    g = bid % n_groups;
    tb = bid / n_groups;
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t read_lane(uint32_t v, int q) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, q);
}

// Raw buffer over [p, p + bytes): a load takes a per-lane VGPR offset and a
// wave-uniform SGPR offset, so a gathered weight row costs no per-lane address
// arithmetic.  The hardware checks the per-lane offset against `bytes`: a lane
// whose offset lies past the end reads zeros instead of touching memory.
// Every array addressed this way is below 2 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)min(bytes, (size_t)0x7FFFFFFF),
                                           0x00020000);
}

// Row offset of a list entry that stands for nothing (padding, or a lane past
// the end of a list): past every buffer above, so its load returns zeros and
// a non-finite weight elsewhere cannot leak in through a 0 * w product.
constexpr uint32_t NO_ROW = 0x80000000u;
template <class V>
__device__ __forceinline__ V buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <>
__device__ __forceinline__ uint32_t buffer_load<uint32_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
template <>
__device__ __forceinline__ u32x2_t buffer_load<u32x2_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}
template <>
__device__ __forceinline__ u32x4_t buffer_load<u32x4_t>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// Dot product of one 16-byte chunk pair, fp32 accumulation.
__device__ __forceinline__ float dot16(const u32x4_t &a, const u32x4_t &b, float acc, uint16_t) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  // Copy each element to a scalar first: bit-casting a vector element
  // expression directly reads the vector's first element with this compiler.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t ae = a[e], be = b[e];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ae), __builtin_bit_cast(bf16x2_t, be), acc,
                                          false);
  }
  return acc;
}
__device__ __forceinline__ float dot16(const u32x4_t &a, const u32x4_t &b, float acc, float) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(a[e]), __uint_as_float(b[e]), acc);
  return acc;
}

#define TWELL_ROW_SUM_DPP(v)                                                                                   \
  do {                                                                                                         \
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  /* quad_perm 1,0,3,2 */ \
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  /* quad_perm 2,3,0,1 */ \
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)); /* row_ror 4 */        \
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)); /* row_ror 8 */        \
  } while (0)

// Joint wave reduction of U partial-sum registers (one entry each, 64 lanes).
// v_permlane32_swap / v_permlane16_swap fold the halves and quarters of the
// wave of two registers into one, then DPP sums each 16-lane row; every lane
// of row r ends up with the total of entry Reduce<U>::entry(r).
template <int U> struct Reduce;
template <>
struct Reduce<4> {
  __device__ __forceinline__ static int entry(int row) { return ((row & 1) << 1) | (row >> 1); }
  __device__ __forceinline__ static float run(const float (&p)[4]) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[2]), __float_as_uint(p[3]), false, false);
    const float s01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // lanes 0-31: entry 0, 32-63: entry 1
    const float s23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
    float v = __uint_as_float(c[0]) + __uint_as_float(c[1]);  // rows: entries 0, 2, 1, 3
    TWELL_ROW_SUM_DPP(v);
    return v;
  }
};
template <>
struct Reduce<1> {
  __device__ __forceinline__ static int entry(int) { return 0; }
  __device__ __forceinline__ static float run(const float (&p)[1]) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[0]), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // halves added
    auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    float v = __uint_as_float(c[0]) + __uint_as_float(c[1]);  // every row: the whole wave
    TWELL_ROW_SUM_DPP(v);
    return v;
  }
};
template <>
struct Reduce<2> {
  __device__ __forceinline__ static int entry(int row) { return row >> 1; }
  __device__ __forceinline__ static float run(const float (&p)[2]) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[1]), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // lanes 0-31: entry 0, 32-63: entry 1
    auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    float v = __uint_as_float(c[0]) + __uint_as_float(c[1]);  // rows: entries 0, 0, 1, 1
    TWELL_ROW_SUM_DPP(v);
    return v;
  }
};

}  // namespace twell
