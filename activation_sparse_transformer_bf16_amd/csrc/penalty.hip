// The L1 activation penalty of the training recipe (gist.science "Sparser,
// Faster, Lighter Transformer Language Models", Resumen Técnico §2.B,
// training-strategy paragraph; §4 gives the coefficient 2e-5), computed from
// TwELL without expanding the activations:
//
//   k_l1_partial: ||h||_1 = sum of the used TwELL slots of rows that did not
//                 overflow plus the dense backup rows of those that did; one
//                 wave per row (lanes over tiles), float64 sums, one partial
//                 per workgroup in a fixed order.
//   k_l1_final:   the partials summed in a fixed order (deterministic).
//   k_l1_grad:    d(lam ||h||_1)/dh in the TwELL matrix's own pattern: lam
//                 (rounded to the storage dtype) in every used slot, 0 in the
//                 padding, lam at the active entries of the dense backup rows.
#include "launch.hpp"

namespace twell {

constexpr int L1_THREADS = 256;
constexpr int L1_WAVES = L1_THREADS / 64;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Rows of one wave: lanes take tiles (a chunk of 64 tiles at a time); a lane
// adds the used slots of its tile.  Rows that overflowed are skipped here and
// summed from the dense backup below.  Every sum runs in a fixed order: per
// lane in slot order, across lanes in a fixed butterfly, across waves and
// workgroups in index order.
template <Dt D>
__global__ __launch_bounds__(L1_THREADS) void k_l1_partial(const uint16_t *__restrict__ cnt,
                                                          const typename DtT<D>::T *__restrict__ val,
                                                          const int *__restrict__ n_ovf, int ovf_cap,
                                                          const typename DtT<D>::T *__restrict__ dense, int T, int F,
                                                          int tile, int cap, double *__restrict__ partial) {
  __shared__ double wsum[L1_WAVES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = F / tile;
  double acc = 0.0;
  for (int t = blockIdx.x * L1_WAVES + wave; t < T; t += gridDim.x * L1_WAVES) {
    const uint16_t *crow = cnt + (size_t)t * nt;
    bool over = false;
    double row = 0.0;
    for (int kb = 0; kb < nt; kb += 64) {
      const int k = kb + lane;
      const int c = k < nt ? (int)crow[k] : 0;
      over |= c > cap;
      const typename DtT<D>::T *v = val + ((size_t)t * nt + k) * cap;
      for (int s = 0; s < min(c, cap); ++s) row += (double)to_f32(v[s]);
    }
    if (ballot(over) == 0) acc += row;
  }
  // dense backup rows (ReLU'd, so every entry is >= 0)
  const int nd = min(*n_ovf, ovf_cap);
  for (int r = blockIdx.x * L1_WAVES + wave; r < nd; r += gridDim.x * L1_WAVES)
    for (int j = lane; j < F; j += 64) acc += (double)to_f32(dense[(size_t)r * F + j]);
  acc = wave_sum_f64(acc);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double b = 0.0;
    for (int w = 0; w < L1_WAVES; ++w) b += wsum[w];
    partial[blockIdx.x] = b;
  }
}

// One wave: lane l adds partials l, l + 64, ... in order (loaded 8 at a time,
// so the loads do not wait for each other), then a fixed butterfly across
// the lanes.
__global__ void k_l1_final(const double *__restrict__ partial, int n, double *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  for (int i0 = 0; i0 < n; i0 += 8 * 64) {
    double v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = i0 + q * 64 + lane;
      v[q] = i < n ? partial[i] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[q];
  }
  s = wave_sum_f64(s);
  if (lane == 0) *out = s;
}

// One thread per (row, tile): its cap slots get lam or +0.
template <Dt D>
__global__ __launch_bounds__(L1_THREADS) void k_l1_grad(const uint16_t *__restrict__ cnt,
                                                       const int *__restrict__ n_ovf, int ovf_cap,
                                                       const typename DtT<D>::T *__restrict__ dense, int T, int F,
                                                       int tile, int cap, float lam,
                                                       typename DtT<D>::T *__restrict__ grad_val,
                                                       typename DtT<D>::T *__restrict__ grad_dense) {
  using TT = typename DtT<D>::T;
  const TT g = from_f32<D>(lam);
  const int nt = F / tile;
  const size_t n_tiles = (size_t)T * nt;
  const size_t stride = (size_t)gridDim.x * L1_THREADS;
  for (size_t tk = (size_t)blockIdx.x * L1_THREADS + threadIdx.x; tk < n_tiles; tk += stride) {
    const int c = min((int)cnt[tk], cap);
    TT *gv = grad_val + tk * cap;
    for (int s = 0; s < cap; ++s) gv[s] = s < c ? g : TT(0);
  }
  if (grad_dense != nullptr) {
    const size_t n_dense = (size_t)min(*n_ovf, ovf_cap) * F;
    for (size_t i = (size_t)blockIdx.x * L1_THREADS + threadIdx.x; i < n_dense; i += stride)
      grad_dense[i] = active_bits(dense[i]) ? g : TT(0);
  }
}

template <Dt D>
static hipError_t launch_l1_norm(const L1Args &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  hipLaunchKernelGGL(k_l1_partial<D>, dim3(L1_BLOCKS), dim3(L1_THREADS), 0, s, a.cnt, (const TT *)a.val, a.n_ovf,
                     a.ovf_cap, (const TT *)a.dense, a.T, a.F, a.tile, a.cap, a.partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_l1_final, dim3(1), dim3(64), 0, s, a.partial, L1_BLOCKS, a.out);
  return hipGetLastError();
}

template <Dt D>
static hipError_t launch_l1_grad(const L1Args &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  hipLaunchKernelGGL(k_l1_grad<D>, dim3(L1_BLOCKS), dim3(L1_THREADS), 0, s, a.cnt, a.n_ovf, a.ovf_cap,
                     (const TT *)a.dense, a.T, a.F, a.tile, a.cap, a.lam, (TT *)a.grad_val, (TT *)a.grad_dense);
  return hipGetLastError();
}

hipError_t l1_norm(const L1Args &a, hipStream_t s) {
  return a.dtype == Dt::BF16 ? launch_l1_norm<Dt::BF16>(a, s) : launch_l1_norm<Dt::F32>(a, s);
}

hipError_t l1_grad(const L1Args &a, hipStream_t s) {
  if (a.T <= 0 && a.grad_dense == nullptr) return hipSuccess;
  return a.dtype == Dt::BF16 ? launch_l1_grad<Dt::BF16>(a, s) : launch_l1_grad<Dt::F32>(a, s);
}

}  // namespace twell
