// Standalone TwELL packing of an explicit pre-activation matrix, and the copy
// of the overflowing rows into the dense backup matrix.
//
// Format: gist.science "Sparser, Faster, Lighter Transformer Language Models",
// Resumen Técnico §2.A (column tiles, per-tile non-zeros; rows that overflow
// go to a dense backup matrix).  One wave packs one row, tile by tile: every
// lane holds tile/64 consecutive columns, per-column activity ballots give the
// ascending rank of each non-zero (mbcnt over the ballots of all lanes below
// plus the lane's own earlier columns), and the first `cap` land in the slots.
// The pass streams the matrix once from HBM.
#include "launch.hpp"

namespace twell {

template <class TT, int EPL> struct LaneVec;
template <> struct LaneVec<uint16_t, 2> { using V = uint32_t; };
template <> struct LaneVec<uint16_t, 4> { using V = u32x2_t; };
template <> struct LaneVec<float, 2> { using V = u32x2_t; };
template <> struct LaneVec<float, 4> { using V = u32x4_t; };

template <class TT, int EPL>
__device__ __forceinline__ void unpack_lane(const typename LaneVec<TT, EPL>::V &v, TT (&o)[EPL]) {
  const uint32_t *w = reinterpret_cast<const uint32_t *>(&v);
  if constexpr (sizeof(TT) == 2) {
#pragma unroll
    for (int e = 0; e < EPL / 2; ++e) {
      o[2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      o[2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = __uint_as_float(w[e]);
  }
}

constexpr int PACK_THREADS = 256;
constexpr int PACK_UNROLL = 4;  // tiles loaded ahead per wave

template <Dt D, int TILE>
__global__ __launch_bounds__(PACK_THREADS) void k_pack(const typename DtT<D>::T *__restrict__ pre, int T, int F,
                                                      int cap, uint16_t *__restrict__ cnt,
                                                      typename DtT<D>::T *__restrict__ val,
                                                      uint8_t *__restrict__ idx) {
  using TT = typename DtT<D>::T;
  constexpr int EPL = TILE / 64;
  using V = typename LaneVec<TT, EPL>::V;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * (PACK_THREADS / 64) + wave;
  if (t >= T) return;
  const int nt = F / TILE;
  const TT *row = pre + (size_t)t * F + lane * EPL;
  for (int kb = 0; kb < nt; kb += PACK_UNROLL) {
    V raw[PACK_UNROLL];
#pragma unroll
    for (int u = 0; u < PACK_UNROLL; ++u)
      if (kb + u < nt) raw[u] = *reinterpret_cast<const V *>(row + (size_t)(kb + u) * TILE);
#pragma unroll
    for (int u = 0; u < PACK_UNROLL; ++u) {
      const int k = kb + u;
      if (k >= nt) break;
      TT v[EPL];
      unpack_lane<TT, EPL>(raw[u], v);
      bool act[EPL];
      int below = 0, total = 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        act[e] = active_bits(v[e]);
        const uint64_t m = ballot(act[e]);
        below += mbcnt(m);
        total += popc64(m);
      }
      const size_t slot0 = ((size_t)t * nt + k) * cap;
      int r = below;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if (act[e]) {
          if (r < cap) {
            val[slot0 + r] = v[e];
            idx[slot0 + r] = (uint8_t)(lane * EPL + e);
          }
          ++r;
        }
      }
      if (lane == 0) cnt[(size_t)t * nt + k] = (uint16_t)total;
      for (int s = lane; s < cap; s += 64) {
        if (s >= total) {
          val[slot0 + s] = TT(0);
          idx[slot0 + s] = 0;
        }
      }
    }
  }
}

template <Dt D, int TILE>
static hipError_t launch_pack(const PackArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int blocks = (a.T + PACK_THREADS / 64 - 1) / (PACK_THREADS / 64);
  hipLaunchKernelGGL((k_pack<D, TILE>), dim3(blocks), dim3(PACK_THREADS), 0, s, (const TT *)a.pre, a.T, a.F,
                     a.cap, a.cnt, (TT *)a.val, a.idx);
  return hipGetLastError();
}

hipError_t pack_tiles(const PackArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.dtype == Dt::BF16) {
    if (a.tile == 256) return launch_pack<Dt::BF16, 256>(a, s);
    if (a.tile == 128) return launch_pack<Dt::BF16, 128>(a, s);
  } else {
    if (a.tile == 256) return launch_pack<Dt::F32, 256>(a, s);
    if (a.tile == 128) return launch_pack<Dt::F32, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

// dense[r][:] = ReLU(pre[ovf_rows[r]][:]) for r < min(*n_ovf, ovf_cap).
template <Dt D>
__global__ __launch_bounds__(256) void k_dense_rows(const typename DtT<D>::T *__restrict__ pre, int F,
                                                   const int *__restrict__ ovf_rows, const int *__restrict__ n_ovf,
                                                   int ovf_cap, typename DtT<D>::T *__restrict__ dense) {
  using TT = typename DtT<D>::T;
  const int n = min(*n_ovf, ovf_cap);
  for (int r = blockIdx.x; r < n; r += gridDim.x) {
    const TT *src = pre + (size_t)ovf_rows[r] * F;
    TT *dst = dense + (size_t)r * F;
    for (int j = threadIdx.x; j < F; j += blockDim.x) {
      const TT v = src[j];
      dst[j] = active_bits(v) ? v : TT(0);
    }
  }
}

hipError_t pack_dense_rows(const DenseRowsArgs &a, hipStream_t s) {
  if (a.dense == nullptr || a.ovf_cap <= 0 || a.T <= 0) return hipSuccess;
  const int blocks = std::min(std::min(a.ovf_cap, a.T), 2048);
  if (a.dtype == Dt::BF16)
    hipLaunchKernelGGL(k_dense_rows<Dt::BF16>, dim3(blocks), dim3(256), 0, s, (const uint16_t *)a.pre, a.F,
                       a.ovf_rows, a.n_ovf, a.ovf_cap, (uint16_t *)a.dense);
  else
    hipLaunchKernelGGL(k_dense_rows<Dt::F32>, dim3(blocks), dim3(256), 0, s, (const float *)a.pre, a.F,
                       a.ovf_rows, a.n_ovf, a.ovf_cap, (float *)a.dense);
  return hipGetLastError();
}

}  // namespace twell
