// Device-side helpers shared by the TwELL kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

enum class Dt { F32 = 0, BF16 = 1 };

template <Dt D> struct DtT;
template <> struct DtT<Dt::F32> {
  using T = float;
  static constexpr int size = 4;
};
template <> struct DtT<Dt::BF16> {
  using T = uint16_t;
  static constexpr int size = 2;
};

// ---- storage <-> fp32 -------------------------------------------------------

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// bf16 of the low / high half of a packed dword (exact widening).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round fp32 to bf16, nearest-even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <Dt D> __device__ __forceinline__ typename DtT<D>::T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<Dt::F32>(float f) { return f; }
template <> __device__ __forceinline__ uint16_t from_f32<Dt::BF16>(float f) { return bf16_rne(f); }

// ---- the TwELL activity predicate ------------------------------------------
// A stored value is active iff IEEE v > 0, decided on its bits.
__device__ __forceinline__ bool active_bits(float v) {
  int32_t b = __float_as_int(v);
  return b > 0 && b <= 0x7F800000;
}
__device__ __forceinline__ bool active_bits(uint16_t v) {
  int32_t b = (int16_t)v;
  return b > 0 && b <= 0x7F80;
}

// Activity of round_to_storage(v) for an fp32 value v, without rounding first.
// fp32 storage: v > 0 (NaN compares false, +inf is active).
// bf16 storage: round-to-nearest-even of v is > 0 iff v > 2^-134 (the half
// quantum of the smallest bf16 denormal ties to +0); +inf is active, NaN not.
template <Dt D> __device__ __forceinline__ bool active_after_round(float v);
template <> __device__ __forceinline__ bool active_after_round<Dt::F32>(float v) { return v > 0.0f; }
template <> __device__ __forceinline__ bool active_after_round<Dt::BF16>(float v) {
  return v > 0x1p-134f;
}

// ---- wave64 helpers ---------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of m in lanes below the calling lane.
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sum over the 64 lanes of a wave with DPP lane moves (no LDS traffic); the
// total lands in lane 63.  Steps: pairs and quads (quad_perm), 8 and 16 lanes
// (row_ror 4, 8), then rows 0+1 and 2+3 (row_bcast15 into rows 1 and 3) and
// all four rows (row_bcast31 into rows 2 and 3).
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
#define TWELL_DPP_ADD(CTRL, ROWS) \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false))
  TWELL_DPP_ADD(0xB1, 0xF);   // quad_perm 1,0,3,2
  TWELL_DPP_ADD(0x4E, 0xF);   // quad_perm 2,3,0,1
  TWELL_DPP_ADD(0x124, 0xF);  // row_ror 4
  TWELL_DPP_ADD(0x128, 0xF);  // row_ror 8
  TWELL_DPP_ADD(0x142, 0xA);  // row_bcast15 into rows 1, 3
  TWELL_DPP_ADD(0x143, 0xC);  // row_bcast31 into rows 2, 3
#undef TWELL_DPP_ADD
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (integers), with DPP row
// shifts inside each 16-lane row and row broadcasts across rows; every lane of
// the wave must be active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr 1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr 2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr 4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr 8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast31 into rows 2, 3
  return v;
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X
// (blockIdx.x % 8 is the XCD).  Remap a linear block id so that consecutive
// remapped ids land on the same XCD, sharing its L2.  Identity when the grid
// is not a multiple of 8.
__device__ __forceinline__ int xcd_linear(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

}  // namespace twell
