// Dense ReGLU FFN on the matrix cores: the dense-backup path of the hybrid
// format (rows whose TwELL tiles overflowed; gist.science "Sparser, Faster,
// Lighter Transformer Language Models", Resumen Técnico §2.A, and the
// q2bstudio post on TwELL, third paragraph) and the dense baseline layer.
//
//   k_gate_up: one matmul over W_g and W_u rows of the same 128 hidden units,
//              interleaved by 32 so that each lane holds the gate and the up
//              value of a unit; epilogue a = ReLU(round(pre)) * u, rounded to
//              the storage dtype (and optionally h = ReLU(round(pre)) stored).
//   k_down:    y = a W_d with W_d [F][d] read n-contiguous and transposed into
//              the k-contiguous LDS layout of the mainloop.
// Rows may be gathered through an index list whose length lives on the device;
// workgroups past that length return before loading anything.
#include "gemm.hpp"
#include "launch.hpp"

#include <algorithm>

namespace twell {

template <Dt D>
__device__ __forceinline__ void gate_up_tile(
    int bid, const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wg,
    const typename DtT<D>::T *__restrict__ wu, const float *__restrict__ beta, int M, int K, int F,
    const int *__restrict__ rows, const int *__restrict__ n_rows_dev, typename DtT<D>::T *__restrict__ a_ws,
    typename DtT<D>::T *__restrict__ h_out, int h_cap) {
  using T = typename DtT<D>::T;
  constexpr int BN = 256, UNITS = 128;  // B tile: 128 hidden units, each as a W_g row and a W_u row
  using WT = WaveTile<BN>;
  constexpr int NWM = WT::NWM;
  static_assert(WT::NWN == 2, "a wave holds one gate block and one up block");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int mt = (M + GEMM_BM - 1) / GEMM_BM, ntl = F / UNITS;
  int tm, tn;
  tile_coords(bid, mt, ntl, tm, tn);
  const int m0 = tm * GEMM_BM, n0 = tn * UNITS;
  const int n_eff = n_rows_dev ? min(*n_rows_dev, M) : M;
  if (m0 >= n_eff) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = WT::row0(wave), col0 = WT::col0(wave);
  const size_t ldk = (size_t)K * sizeof(T);
  auto phys = [&](int r) { return rows ? rows[r] : r; };

  auto rowA = [&](int r) {
    const int lr = m0 + r;
    const int row = lr < n_eff ? phys(lr) : phys(0);
    return reinterpret_cast<const char *>(x) + (size_t)row * ldk;
  };
  // B row r: 64-row group g = r / 64 covers units n0 + 32g .. n0 + 32g + 31,
  // first as W_g rows, then as W_u rows, so the wave that owns columns
  // [64g, 64g + 64) holds the gate and the up value of the same unit in the
  // same lane (accumulator blocks 0 and 1).
  auto rowB = [&](int r) {
    const T *w = (r & 32) ? wu : wg;
    return reinterpret_cast<const char *>(w) + (size_t)(n0 + 32 * (r >> 6) + (r & 31)) * ldk;
  };

  auto rowv = [&](int r) -> const float * {
    return beta != nullptr ? beta + phys(min(m0 + r, n_eff - 1)) : nullptr;
  };
  auto init = [&](f32x16_t (&a)[NWM][2], const float *vals) {
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm) {
#pragma unroll
      for (int i = 0; i < 16; ++i) a[bm][0][i] = vals != nullptr ? vals[acc_row(row0, bm, i, lane)] : 0.0f;
      a[bm][1] = f32x16_t{};
    }
  };
  f32x16_t acc[NWM][2];
  gemm_mainloop_dma<D, BN>(acc, rowA, rowB, rowv, init, (int)(ldk / SLAB), smem);

  const int col = lane & 31;
  int row_base = m0 + row0 + 4 * (lane >> 5);  // opaque: keep row math after the mainloop
  asm volatile("" : "+v"(row_base));
  const size_t j = (size_t)n0 + col0 / 2 + col;
#pragma unroll
  for (int bm = 0; bm < NWM; ++bm) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int lr = row_base + 32 * bm + 8 * (i >> 2) + (i & 3);
      if (lr >= n_eff) continue;
      const T hb = from_f32<D>(acc[bm][0][i]);
      const bool act = active_bits(hb);
      const float h = act ? to_f32(hb) : 0.0f;
      a_ws[(size_t)lr * F + j] = from_f32<D>(h * acc[bm][1][i]);
      if (h_out != nullptr && lr < h_cap) h_out[(size_t)lr * F + j] = act ? hb : T(0);
    }
  }
}

template <Dt D>
__device__ __forceinline__ void down_tile(
    int bid, const typename DtT<D>::T *__restrict__ a_ws, const typename DtT<D>::T *__restrict__ wd, int M, int K,
    int N, const int *__restrict__ rows, const int *__restrict__ n_rows_dev,
    typename DtT<D>::T *__restrict__ y) {
  using T = typename DtT<D>::T;
  constexpr int BN = 256;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int mt = (M + GEMM_BM - 1) / GEMM_BM, ntl = N / BN;
  int tm, tn;
  tile_coords(bid, mt, ntl, tm, tn);
  const int m0 = tm * GEMM_BM, n0 = tn * BN;
  const int n_eff = n_rows_dev ? min(*n_rows_dev, M) : M;
  if (m0 >= n_eff) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t ldk = (size_t)K * sizeof(T);

  KRowLoader<GEMM_BM> la;
  la.init(tid, [&](int r) {
    int lr = min(m0 + r, n_eff - 1);
    return reinterpret_cast<const char *>(a_ws) + (size_t)lr * ldk;
  });
  NColLoader<D, BN> lb;
  lb.init(tid, wd, (size_t)N * sizeof(T), n0);

  f32x16_t acc[2][8];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < 8; ++bn) acc[bm][bn] = f32x16_t{};

  gemm_mainloop<D, BN>(acc, la, lb, K / (KCHUNK_BYTES / (int)sizeof(T)), smem);

  const int col = lane & 31;
  int row_base = m0 + 64 * wave + 4 * (lane >> 5);  // opaque: keep row math after the mainloop
  asm volatile("" : "+v"(row_base));
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int lr = row_base + 32 * bm + 8 * (i >> 2) + (i & 3);
      if (lr >= n_eff) continue;
      const size_t prow = rows ? (size_t)rows[lr] : (size_t)lr;
#pragma unroll
      for (int bn = 0; bn < 8; ++bn) y[prow * N + n0 + 32 * bn + col] = from_f32<D>(acc[bm][bn][i]);
    }
  }
}

// Each workgroup takes tiles bid, bid + gridDim.x, ...: the dense baseline
// launches one workgroup per tile, the fallback (row count on the device) a
// grid of at most FALLBACK_WGS, so that an empty fallback costs little.
constexpr int FALLBACK_WGS = 256;

template <Dt D>
__global__ __launch_bounds__(DMA_THREADS) void k_gate_up(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wg,
    const typename DtT<D>::T *__restrict__ wu, const float *__restrict__ beta, int M, int K, int F,
    const int *__restrict__ rows, const int *__restrict__ n_rows_dev, typename DtT<D>::T *__restrict__ a_ws,
    typename DtT<D>::T *__restrict__ h_out, int h_cap) {
  const int tiles = (M + GEMM_BM - 1) / GEMM_BM * (F / 128);
  for (int bid = blockIdx.x; bid < tiles; bid += gridDim.x)
    gate_up_tile<D>(bid, x, wg, wu, beta, M, K, F, rows, n_rows_dev, a_ws, h_out, h_cap);
}

template <Dt D, bool LOOP>
__global__ __launch_bounds__(GEMM_THREADS) void k_down(
    const typename DtT<D>::T *__restrict__ a_ws, const typename DtT<D>::T *__restrict__ wd, int M, int K,
    int N, const int *__restrict__ rows, const int *__restrict__ n_rows_dev,
    typename DtT<D>::T *__restrict__ y) {
  if constexpr (LOOP) {
    const int tiles = (M + GEMM_BM - 1) / GEMM_BM * (N / 256);
    for (int bid = blockIdx.x; bid < tiles; bid += gridDim.x)
      down_tile<D>(bid, a_ws, wd, M, K, N, rows, n_rows_dev, y);
  } else {
    down_tile<D>(blockIdx.x, a_ws, wd, M, K, N, rows, n_rows_dev, y);
  }
}

template <Dt D>
static hipError_t launch_gate_up(const DenseArgs &a, hipStream_t s) {
  using T = typename DtT<D>::T;
  auto kern = k_gate_up<D>;
  const int lds = gemm_dma_lds_bytes(256);
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int mt = (a.M + GEMM_BM - 1) / GEMM_BM, ntl = a.F / 128;
  const int grid = a.n_rows_dev ? std::min(mt * ntl, FALLBACK_WGS) : mt * ntl;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(DMA_THREADS), lds, s, (const T *)a.x, (const T *)a.wg,
                     (const T *)a.wu, a.beta, a.M, a.d, a.F, a.rows, a.n_rows_dev, (T *)a.a_ws,
                     (T *)a.h_out, a.h_cap);
  return hipGetLastError();
}

template <Dt D>
static hipError_t launch_down(const DenseArgs &a, hipStream_t s) {
  using T = typename DtT<D>::T;
  auto kern = a.n_rows_dev ? k_down<D, true> : k_down<D, false>;
  const int lds = gemm_lds_bytes(256);
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int mt = (a.M + GEMM_BM - 1) / GEMM_BM, ntl = a.d / 256;
  const int grid = a.n_rows_dev ? std::min(mt * ntl, FALLBACK_WGS) : mt * ntl;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(GEMM_THREADS), lds, s, (const T *)a.a_ws, (const T *)a.wd,
                     a.M, a.F, a.d, a.rows, a.n_rows_dev, (T *)a.y);
  return hipGetLastError();
}

hipError_t dense_gate_up(const DenseArgs &a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  return a.dtype == Dt::BF16 ? launch_gate_up<Dt::BF16>(a, s) : launch_gate_up<Dt::F32>(a, s);
}

hipError_t dense_down(const DenseArgs &a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  return a.dtype == Dt::BF16 ? launch_down<Dt::BF16>(a, s) : launch_down<Dt::F32>(a, s);
}

}  // namespace twell
