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
// workgroups past that length return before loading anything.  For that
// fallback, when the rows fill fewer output tiles than the grid has
// workgroups, K is split into S ranges so that tiles * S work items keep the
// grid busy: each item writes an fp32 partial tile, and a reduction kernel
// adds the S partials in K order and applies the epilogue.
#include "gemm.hpp"
#include "launch.hpp"
#include "part_index.hpp"

#include <algorithm>

namespace twell {

constexpr int SPLIT_TILE = FALLBACK_SPLIT_TILE;
static_assert(SPLIT_TILE == GEMM_BM * 256, "a partial tile is one 256 x 256 output tile");

// K ranges per output tile (fallback_split): enough to give every workgroup
// of the grid a work item, at most GATE_UP_SPLIT_MAX / DOWN_SPLIT_MAX.  The
// limits are measured: each K range adds a 256 KB fp32 partial tile written
// and read back, and past 2 ranges (gate+up, K = d) or 16 (down, K = d_ff)
// that traffic costs more than the idle workgroups it would fill.
constexpr int REDUCE_BATCH = 8;  // partials loaded together by the reduction kernels (added in K order)

// One 256-row x 128-unit tile (tm, tn) of the gate / up matmul over K slabs
// [k0, k0 + nk).  part == null: the epilogue writes a (and h); otherwise the
// raw fp32 accumulators go to the partial tile part[row][col] (no bias).
template <Dt D>
__device__ __forceinline__ void gate_up_tile(
    int tm, int tn, int k0, int nk, float *__restrict__ part, const typename DtT<D>::T *__restrict__ x,
    const typename DtT<D>::T *__restrict__ wg, const typename DtT<D>::T *__restrict__ wu,
    const float *__restrict__ beta, int M, int K, int F, const int *__restrict__ rows, int n_eff,
    typename DtT<D>::T *__restrict__ a_ws, typename DtT<D>::T *__restrict__ h_out, int h_cap) {
  using T = typename DtT<D>::T;
  constexpr int BN = 256, UNITS = 128;  // B tile: 128 hidden units, each as a W_g row and a W_u row
  using WT = WaveTile<BN>;
  constexpr int NWM = WT::NWM;
  static_assert(WT::NWN == 2, "a wave holds one gate block and one up block");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int m0 = tm * GEMM_BM, n0 = tn * UNITS;
  if (m0 >= n_eff) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = WT::row0(wave), col0 = WT::col0(wave);
  const size_t ldk = (size_t)K * sizeof(T);
  auto phys = [&](int r) { return rows ? rows[r] : r; };

  const size_t koff = (size_t)k0 * SLAB;
  auto rowA = [&](int r) {
    const int lr = m0 + r;
    const int row = lr < n_eff ? phys(lr) : phys(0);
    return reinterpret_cast<const char *>(x) + (size_t)row * ldk + koff;
  };
  // B row r: 64-row group g = r / 64 covers units n0 + 32g .. n0 + 32g + 31,
  // first as W_g rows, then as W_u rows, so the wave that owns columns
  // [64g, 64g + 64) holds the gate and the up value of the same unit in the
  // same lane (accumulator blocks 0 and 1).
  auto rowB = [&](int r) {
    const T *w = (r & 32) ? wu : wg;
    return reinterpret_cast<const char *>(w) + (size_t)(n0 + 32 * (r >> 6) + (r & 31)) * ldk + koff;
  };

  auto rowv = [&](int r) -> const float * {
    return beta != nullptr && part == nullptr ? beta + phys(min(m0 + r, n_eff - 1)) : nullptr;
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
  gemm_mainloop_dma<D, BN, DmaBig>(acc, rowA, rowB, rowv, init, nk, smem);

  const int col = lane & 31;
  if (part != nullptr) {
    float *q = part + (size_t)wave * (NWM * 2 * 16 * 64) + lane;
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm)
#pragma unroll
      for (int bn = 0; bn < 2; ++bn)
#pragma unroll
        for (int i = 0; i < 16; ++i) q[((bm * 2 + bn) * 16 + i) * 64] = acc[bm][bn][i];
    return;
  }
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

// One 256 x BN tile (tm, tn) of y = a W_d over K chunks [k0, k0 + nk) of
// 128 bytes; part == null: y is written, otherwise the fp32 partial tile.
template <Dt D, int BN>
__device__ __forceinline__ void down_tile(
    int tm, int tn, int k0, int nk, float *__restrict__ part, const typename DtT<D>::T *__restrict__ a_ws,
    const typename DtT<D>::T *__restrict__ wd, int M, int K, int N, const int *__restrict__ rows, int n_eff,
    typename DtT<D>::T *__restrict__ y) {
  using T = typename DtT<D>::T;
  constexpr int NB = BN / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int m0 = tm * GEMM_BM, n0 = tn * BN;
  if (m0 >= n_eff) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t ldk = (size_t)K * sizeof(T);

  KRowLoader<GEMM_BM> la;
  la.init(tid, [&](int r) {
    int lr = min(m0 + r, n_eff - 1);
    return reinterpret_cast<const char *>(a_ws) + (size_t)lr * ldk + (size_t)k0 * KCHUNK_BYTES;
  });
  NColLoader<D, BN> lb;
  // chunk kt covers k rows [kt * KCHUNK_BYTES / s, ...) of W_d: start at chunk k0
  lb.init(tid, reinterpret_cast<const char *>(wd) + (size_t)k0 * (KCHUNK_BYTES / sizeof(T)) * N * sizeof(T),
          (size_t)N * sizeof(T), n0);

  f32x16_t acc[2][NB];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < NB; ++bn) acc[bm][bn] = f32x16_t{};

  gemm_mainloop<D, BN>(acc, la, lb, nk, smem);

  const int col = lane & 31;
  if (part != nullptr) {
    float *q = part + (size_t)wave * (2 * NB * 16 * 64) + lane;
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int bn = 0; bn < NB; ++bn)
#pragma unroll
        for (int i = 0; i < 16; ++i) q[((bm * NB + bn) * 16 + i) * 64] = acc[bm][bn][i];
    return;
  }
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
      for (int bn = 0; bn < NB; ++bn) y[prow * N + n0 + 32 * bn + col] = from_f32<D>(acc[bm][bn][i]);
    }
  }
}

// The dense baseline launches one workgroup per tile.  The fallback (row count
// on the device) runs FALLBACK_WGS workgroups over the work items: every tile
// whole when the rows fill the grid, else tiles x S K ranges into partials.
template <Dt D>
__global__ __launch_bounds__(DMA_THREADS) void k_gate_up(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wg,
    const typename DtT<D>::T *__restrict__ wu, const float *__restrict__ beta, int M, int K, int F,
    const int *__restrict__ rows, const int *__restrict__ n_rows_dev, int n_sub,
    typename DtT<D>::T *__restrict__ a_ws, typename DtT<D>::T *__restrict__ h_out, int h_cap,
    float *__restrict__ partial, int partial_tiles) {
  using T = typename DtT<D>::T;
  const int nk = (int)((size_t)K * sizeof(T) / SLAB);
  const int mt = (M + GEMM_BM - 1) / GEMM_BM, ntl = F / 128;
  if (n_rows_dev == nullptr) {
    int tm, tn;
    tile_coords(blockIdx.x, mt, ntl, tm, tn);
    gate_up_tile<D>(tm, tn, 0, nk, nullptr, x, wg, wu, beta, M, K, F, rows, M, a_ws, h_out, h_cap);
    return;
  }
  const int n_eff = min(max(*n_rows_dev - n_sub, 0), M);
  const int tiles = (n_eff + GEMM_BM - 1) / GEMM_BM * ntl;
  const int S = fallback_split(tiles, nk, GATE_UP_SPLIT_MAX, partial_tiles);
  for (int w = blockIdx.x; w < tiles * S; w += gridDim.x) {
    const int tile = w / S, kc = w - tile * S;
    const int k0 = kc * nk / S, k1 = (kc + 1) * nk / S;
    gate_up_tile<D>(tile / ntl, tile % ntl, k0, k1 - k0, S > 1 ? partial + (size_t)w * SPLIT_TILE : nullptr, x,
                    wg, wu, beta, M, K, F, rows, n_eff, a_ws, h_out, h_cap);
  }
}

// The fallback's gate / up epilogue after a split: pre = (sum of the S
// partials in K order) + beta, h = ReLU(round(pre)), a = round(h * u).
template <Dt D>
__global__ __launch_bounds__(256) void k_gate_up_reduce(const float *__restrict__ partial,
                                                        const float *__restrict__ beta, int M, int K, int F,
                                                        const int *__restrict__ rows,
                                                        const int *__restrict__ n_rows_dev, int n_sub,
                                                        typename DtT<D>::T *__restrict__ a_ws,
                                                        typename DtT<D>::T *__restrict__ h_out, int h_cap,
                                                        int partial_tiles) {
  using T = typename DtT<D>::T;
  const int nk = (int)((size_t)K * sizeof(T) / SLAB);
  const int ntl = F / 128;
  const int n_eff = min(max(*n_rows_dev - n_sub, 0), M);
  const int tiles = (n_eff + GEMM_BM - 1) / GEMM_BM * ntl;
  const int S = fallback_split(tiles, nk, GATE_UP_SPLIT_MAX, partial_tiles);
  if (S == 1) return;
  const size_t total = (size_t)tiles * GEMM_BM * 128;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const int tile = (int)(e / (GEMM_BM * 128));
    const int rem = (int)(e - (size_t)tile * GEMM_BM * 128);
    const int r = rem / 128, u = rem % 128;  // tile row, unit within the tile
    const int lr = (tile / ntl) * GEMM_BM + r;
    if (lr >= n_eff) continue;
    const int gcol = 64 * (u >> 5) + (u & 31);  // gate column; the up column is gcol + 32
    const float *p = partial + (size_t)tile * S * SPLIT_TILE;
    const int ig = gate_up_part_index(r, gcol), iu = gate_up_part_index(r, gcol + 32);
    float pre = 0.f, up = 0.f;
    int kc = 0;
    for (; kc + REDUCE_BATCH <= S; kc += REDUCE_BATCH) {  // loads of a batch in flight together
      float qg[REDUCE_BATCH], qu[REDUCE_BATCH];
#pragma unroll
      for (int i = 0; i < REDUCE_BATCH; ++i) {
        qg[i] = p[(size_t)(kc + i) * SPLIT_TILE + ig];
        qu[i] = p[(size_t)(kc + i) * SPLIT_TILE + iu];
      }
#pragma unroll
      for (int i = 0; i < REDUCE_BATCH; ++i) {
        pre += qg[i];
        up += qu[i];
      }
    }
    for (; kc < S; ++kc) {
      pre += p[(size_t)kc * SPLIT_TILE + ig];
      up += p[(size_t)kc * SPLIT_TILE + iu];
    }
    const int prow = rows ? rows[lr] : lr;
    if (beta != nullptr) pre += beta[prow];
    const T hb = from_f32<D>(pre);
    const bool act = active_bits(hb);
    const float h = act ? to_f32(hb) : 0.0f;
    const size_t j = (size_t)(tile % ntl) * 128 + u;
    a_ws[(size_t)lr * F + j] = from_f32<D>(h * up);
    if (h_out != nullptr && lr < h_cap) h_out[(size_t)lr * F + j] = act ? hb : T(0);
  }
}

// Output tiles of BN columns; the fallback uses BN = 128 (twice the tiles of
// 256-column ones for the same rows, so a chunk of a few thousand overflow
// rows still fills the grid), the dense baseline BN = 256.  Partial tiles of
// the split hold 256 x BN floats; the area's capacity, given in 256 x 256
// tiles, holds 256 / BN times as many.
template <Dt D, bool LOOP, int BN>
__global__ __launch_bounds__(GEMM_THREADS) void k_down(
    const typename DtT<D>::T *__restrict__ a_ws, const typename DtT<D>::T *__restrict__ wd, int M, int K,
    int N, const int *__restrict__ rows, const int *__restrict__ n_rows_dev, int n_sub,
    typename DtT<D>::T *__restrict__ y, float *__restrict__ partial, int partial_tiles) {
  using T = typename DtT<D>::T;
  const int nk = K / (KCHUNK_BYTES / (int)sizeof(T));
  const int mt = (M + GEMM_BM - 1) / GEMM_BM, ntl = N / BN;
  if constexpr (LOOP) {
    const int n_eff = min(max(*n_rows_dev - n_sub, 0), M);
    const int tiles = (n_eff + GEMM_BM - 1) / GEMM_BM * ntl;
    const int S = fallback_split(tiles, nk, DOWN_SPLIT_MAX, partial_tiles * (256 / BN));
    for (int w = blockIdx.x; w < tiles * S; w += gridDim.x) {
      const int tile = w / S, kc = w - tile * S;
      const int k0 = kc * nk / S, k1 = (kc + 1) * nk / S;
      down_tile<D, BN>(tile / ntl, tile % ntl, k0, k1 - k0,
                       S > 1 ? partial + (size_t)w * GEMM_BM * BN : nullptr, a_ws, wd, M, K, N, rows, n_eff, y);
    }
  } else {
    int tm, tn;
    tile_coords(blockIdx.x, mt, ntl, tm, tn);
    down_tile<D, BN>(tm, tn, 0, nk, nullptr, a_ws, wd, M, K, N, rows, M, y);
  }
}

// y rows of the fallback after a split: the S partials added in K order.
template <Dt D, int BN>
__global__ __launch_bounds__(256) void k_down_reduce(const float *__restrict__ partial, int M, int K, int N,
                                                     const int *__restrict__ rows,
                                                     const int *__restrict__ n_rows_dev, int n_sub,
                                                     typename DtT<D>::T *__restrict__ y, int partial_tiles) {
  using T = typename DtT<D>::T;
  constexpr int PT = GEMM_BM * BN;  // floats of one partial tile
  const int nk = K / (KCHUNK_BYTES / (int)sizeof(T));
  const int ntl = N / BN;
  const int n_eff = min(max(*n_rows_dev - n_sub, 0), M);
  const int tiles = (n_eff + GEMM_BM - 1) / GEMM_BM * ntl;
  const int S = fallback_split(tiles, nk, DOWN_SPLIT_MAX, partial_tiles * (256 / BN));
  if (S == 1) return;
  const size_t total = (size_t)tiles * PT;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const int tile = (int)(e / PT);
    const int rem = (int)(e - (size_t)tile * PT);
    const int r = rem / BN, c = rem % BN;
    const int lr = (tile / ntl) * GEMM_BM + r;
    if (lr >= n_eff) continue;
    const float *p = partial + (size_t)tile * S * PT + down_part_index<BN>(r, c);
    float v = 0.f;
    int kc = 0;
    for (; kc + REDUCE_BATCH <= S; kc += REDUCE_BATCH) {  // loads of a batch in flight together
      float q[REDUCE_BATCH];
#pragma unroll
      for (int i = 0; i < REDUCE_BATCH; ++i) q[i] = p[(size_t)(kc + i) * PT];
#pragma unroll
      for (int i = 0; i < REDUCE_BATCH; ++i) v += q[i];
    }
    for (; kc < S; ++kc) v += p[(size_t)kc * PT];
    const size_t prow = rows ? (size_t)rows[lr] : (size_t)lr;
    y[prow * N + (size_t)(tile % ntl) * BN + c] = from_f32<D>(v);
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
  const int grid = a.n_rows_dev ? FALLBACK_WGS : mt * ntl;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(DMA_THREADS), lds, s, (const T *)a.x, (const T *)a.wg,
                     (const T *)a.wu, a.beta, a.M, a.d, a.F, a.rows, a.n_rows_dev, a.n_sub, (T *)a.a_ws,
                     (T *)a.h_out, a.h_cap, a.partial, a.partial_tiles);
  e = hipGetLastError();
  // the reduction runs only where a split is possible (it exits when S == 1)
  if (e != hipSuccess || a.n_rows_dev == nullptr || a.partial_tiles < 2) return e;
  hipLaunchKernelGGL(k_gate_up_reduce<D>, dim3(1024), dim3(256), 0, s, (const float *)a.partial, a.beta, a.M, a.d,
                     a.F, a.rows, a.n_rows_dev, a.n_sub, (T *)a.a_ws, (T *)a.h_out, a.h_cap, a.partial_tiles);
  return hipGetLastError();
}

template <Dt D>
static hipError_t launch_down(const DenseArgs &a, hipStream_t s) {
  using T = typename DtT<D>::T;
  constexpr int BNF = FALLBACK_DOWN_BN;
  auto kern = a.n_rows_dev ? k_down<D, true, BNF> : k_down<D, false, 256>;
  const int lds = gemm_lds_bytes(a.n_rows_dev ? BNF : 256);
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int mt = (a.M + GEMM_BM - 1) / GEMM_BM, ntl = a.d / 256;
  const int grid = a.n_rows_dev ? FALLBACK_WGS : mt * ntl;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(GEMM_THREADS), lds, s, (const T *)a.a_ws, (const T *)a.wd,
                     a.M, a.F, a.d, a.rows, a.n_rows_dev, a.n_sub, (T *)a.y, a.partial, a.partial_tiles);
  e = hipGetLastError();
  if (e != hipSuccess || a.n_rows_dev == nullptr || a.partial_tiles < 1) return e;
  hipLaunchKernelGGL((k_down_reduce<D, BNF>), dim3(1024), dim3(256), 0, s, (const float *)a.partial, a.M, a.F,
                     a.d, a.rows, a.n_rows_dev, a.n_sub, (T *)a.y, a.partial_tiles);
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
