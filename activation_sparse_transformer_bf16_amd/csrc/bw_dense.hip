// Backward of the hybrid format's dense backup rows on the matrix cores: the
// hybrid-times-dense and dense-times-hybrid products of gist.science
// "Sparser, Faster, Lighter Transformer Language Models", Resumen Técnico
// §2.B, for the rows the hybrid format of §2.A keeps dense.  For the R stored
// dense rows t_r (the ascending dense row list) with backup rows h_r:
//
//   U = X_R W_u^T,  DA = DY_R W_d^T                      k_bwd_ud ([R][F] each)
//   on active entries: a = h U, du = DA h, dpre = DA U + lam; 0 elsewhere
//   dx_R = du W_u + dpre W_g                             k_bwd_dx (+ k_bwd_dx_reduce)
//   dW_g += dpre^T X_R, dW_u += du^T X_R, dW_d += a^T DY_R   k_bwd_dw
//
// The entry kernels skip these rows (their lists are empty there).  On the
// same stream: k_bwd_dx runs after the entry kernels' dx (which writes zero
// rows for them) and overwrites those rows; k_bwd_dw runs before the entry
// kernels' weight gradients and writes the dense rows' part, to which that
// kernel then adds the other rows' sums.
//
// Operands.  U and DA are products of stored values (x, dy, weights), taken
// on the matrix cores with fp32 accumulation like every other product here.
// The dx product takes du and dpre rounded to the storage dtype (dx itself is
// rounded once to it).  The weight-gradient products keep fp32 precision: in
// bf16 each of a, du, dpre is split into a high part bf16(v) and a low part
// bf16(v - high), whose sum carries v to within 2^-17 of |v|, and both parts
// are multiplied (the K dimension holds the high parts of all R rows, then
// the low parts, against two copies of the gathered x or dy rows); fp32
// operands are used as they are.  Every sum has a fixed order: the results
// are deterministic.
#include "gemm.hpp"
#include "launch.hpp"
#include "part_index.hpp"

#include <algorithm>

namespace twell {

template <Dt D>
struct BwdK {
  static constexpr int KC = KCHUNK_BYTES / DtT<D>::size;  // K elements per chunk of the register-staged mainloop
  static constexpr int NS = D == Dt::BF16 ? 2 : 1;         // parts per value in the weight-gradient products
};

__device__ __forceinline__ int dense_count(const int *n_dense, int cap) { return max(min(*n_dense, cap), 0); }
__host__ __device__ __forceinline__ int pad_to(int v, int m) { return (v + m - 1) / m * m; }

// ---------------------------------------------------------------------------
// Gathered rows of x and dy for the weight-gradient products: NS copies of
// [Rp][d], rows R .. Rp of each copy zero (Rp = R rounded up to whole K
// chunks).

template <Dt D>
__global__ __launch_bounds__(256) void k_bwd_gather(const typename DtT<D>::T *__restrict__ x,
                                                   const typename DtT<D>::T *__restrict__ dy,
                                                   const int *__restrict__ dense_rows, const int *__restrict__ n_dense,
                                                   int dense_cap, int T, int d, typename DtT<D>::T *__restrict__ xr,
                                                   typename DtT<D>::T *__restrict__ dyr) {
  using K = BwdK<D>;
  const int R = dense_count(n_dense, dense_cap), Rp = pad_to(R, K::KC);
  const int nchunk = d * DtT<D>::size / 16;
  for (int q = blockIdx.x; q < K::NS * Rp; q += gridDim.x) {
    const int r = q % Rp;
    const int t = r < R ? min(max(dense_rows[r], 0), T - 1) : -1;
    const u32x4_t *xs = reinterpret_cast<const u32x4_t *>(x + (size_t)max(t, 0) * d);
    const u32x4_t *gs = reinterpret_cast<const u32x4_t *>(dy + (size_t)max(t, 0) * d);
    u32x4_t *xo = reinterpret_cast<u32x4_t *>(xr + (size_t)q * d);
    u32x4_t *go = reinterpret_cast<u32x4_t *>(dyr + (size_t)q * d);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int c = threadIdx.x; c < nchunk; c += 256) {
      xo[c] = t >= 0 ? xs[c] : z;
      go[c] = t >= 0 ? gs[c] : z;
    }
  }
}

// ---------------------------------------------------------------------------
// U and DA in one tile: a workgroup of 8 waves takes 128 dense rows x 128
// hidden units of both products.  The direct-to-LDS mainloop stages, per K
// slab, A = [x rows; dy rows] (256 rows) and B = [W_u rows; W_d rows] (256
// rows), and the waves cover only the two diagonal blocks: waves 0-3 the
// x . W_u block (U), waves 4-7 the dy . W_d block (DA), each wave 64 x 64.
// The DA waves then hand their accumulators to the U waves through LDS, all
// waves stage the tile's h block in LDS with 16-byte loads (one round trip
// instead of one per accumulator register), and the U waves form a, du and
// dpre.

struct DiagCfg : DmaCfg<256, 8, 4> {};
template <>
struct WaveTile<256, DiagCfg> {
  static constexpr int NWM = 2, NWN = 2;
  __device__ __forceinline__ static int row0(int wave) { return (wave >> 2) * 128 + ((wave >> 1) & 1) * 64; }
  __device__ __forceinline__ static int col0(int wave) { return (wave >> 2) * 128 + (wave & 1) * 64; }
};
constexpr int UD_BM = 128, UD_BN = 128;

// Four consecutive rows lr0 .. lr0 + 3 of one column of a transposed operand:
// bf16 high parts at lr0, low parts at Rp + lr0; fp32 values at lr0.
template <Dt D>
__device__ __forceinline__ void store_t4(typename DtT<D>::T *row, int lr0, int Rp, const float (&v)[4]) {
  if constexpr (D == Dt::BF16) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint16_t h = bf16_rne(v[q]);
      const float hf = to_f32(h);
      hi[q] = h;
      lo[q] = __builtin_isfinite(hf) ? bf16_rne(v[q] - hf) : 0u;
    }
    *reinterpret_cast<u32x2_t *>(row + lr0) = u32x2_t{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
    *reinterpret_cast<u32x2_t *>(row + Rp + lr0) = u32x2_t{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
  } else {
    *reinterpret_cast<f32x4_t *>(row + lr0) = f32x4_t{v[0], v[1], v[2], v[3]};
  }
}

template <Dt D>
__global__ __launch_bounds__(DiagCfg::THREADS, DiagCfg::WAVES_PER_SIMD) void k_bwd_ud(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ dy,
    const typename DtT<D>::T *__restrict__ wu, const typename DtT<D>::T *__restrict__ wd,
    const int *__restrict__ dense_rows, const int *__restrict__ n_dense, int dense_cap,
    const typename DtT<D>::T *__restrict__ dense, int T, int d, int F, float lam,
    typename DtT<D>::T *__restrict__ du_rm, typename DtT<D>::T *__restrict__ dp_rm, typename DtT<D>::T *__restrict__ at,
    typename DtT<D>::T *__restrict__ dut, typename DtT<D>::T *__restrict__ dpt, int as_stride) {
  using TT = typename DtT<D>::T;
  using K = BwdK<D>;
  using WT = WaveTile<256, DiagCfg>;
  constexpr int NWM = WT::NWM, NWN = WT::NWN;
  using Acc = AccTile<256, DiagCfg>;
  constexpr int ACC_FLOATS = NWM * NWN * 16 * 64;  // one wave's accumulators
  constexpr int XCH_BYTES = 4 * ACC_FLOATS * 4;     // the DA hand-over
  constexpr int H_BYTES = UD_BM * UD_BN * (int)sizeof(TT);
  static_assert(XCH_BYTES + H_BYTES <= gemm_dma_ring_bytes<DiagCfg>(256), "hand-over and h block fit in the ring");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int R = dense_count(n_dense, dense_cap);
  if (R == 0) return;
  const int Rp = pad_to(R, K::KC);
  const int mt = (R + UD_BM - 1) / UD_BM, ntl = F / UD_BN;
  const size_t ldk = (size_t)d * sizeof(TT);
  const int nk = (int)(ldk / SLAB);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = WT::row0(wave) & 127, col0 = WT::col0(wave) & 127;  // position inside the product's block
  float *xch = reinterpret_cast<float *>(smem) + (size_t)(wave & 3) * ACC_FLOATS + lane;
  TT *hs = reinterpret_cast<TT *>(smem + XCH_BYTES);  // [UD_BM][UD_BN]
  auto none = [](int) -> const float * { return nullptr; };
  auto zero = [](Acc &acc, const float *) {
#pragma unroll
    for (int bm = 0; bm < NWM; ++bm)
#pragma unroll
      for (int bn = 0; bn < NWN; ++bn) acc[bm][bn] = f32x16_t{};
  };
  const int items = mt * ntl;
  for (int w = blockIdx.x; w < items; w += gridDim.x) {
    // the row tiles of one unit tile run side by side, on one XCD when every
    // item has a workgroup of its own (so its weight rows are read into one L2)
    const int L = items <= (int)gridDim.x ? xcd_linear(w, items) : w;
    const int tm = L % mt, tn = L / mt;
    const int m0 = tm * UD_BM, n0 = tn * UD_BN;
    auto phys = [&](int r) { return (size_t)min(max(dense_rows[min(m0 + r, R - 1)], 0), T - 1); };
    auto rowA = [&](int r) {
      return reinterpret_cast<const char *>(r < UD_BM ? x : dy) + phys(r & (UD_BM - 1)) * ldk;
    };
    auto rowB = [&](int r) {
      return reinterpret_cast<const char *>(r < UD_BN ? wu : wd) + (size_t)(n0 + (r & (UD_BN - 1))) * ldk;
    };
    Acc acc;
    gemm_mainloop_dma<D, 256, DiagCfg>(acc, rowA, rowB, none, zero, nk, smem);
    // the h block -> LDS, DA waves -> LDS (the ring is free: the mainloop
    // ends with a barrier)
    {
      constexpr int CPR = UD_BN * (int)sizeof(TT) / 16;  // 16-byte chunks per row
      constexpr int PER = UD_BM * CPR / DiagCfg::THREADS;
      u32x4_t hv[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = threadIdx.x + i * DiagCfg::THREADS, r = c / CPR, k = c % CPR;
        hv[i] = *reinterpret_cast<const u32x4_t *>(dense + (size_t)min(m0 + r, R - 1) * F + n0 +
                                                    k * (16 / (int)sizeof(TT)));
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = threadIdx.x + i * DiagCfg::THREADS, r = c / CPR, k = c % CPR;
        *reinterpret_cast<u32x4_t *>(hs + r * UD_BN + k * (16 / (int)sizeof(TT))) = hv[i];
      }
    }
    if (wave >= 4) {
#pragma unroll
      for (int bm = 0; bm < NWM; ++bm)
#pragma unroll
        for (int bn = 0; bn < NWN; ++bn)
#pragma unroll
          for (int i = 0; i < 16; ++i) xch[((bm * NWN + bn) * 16 + i) * 64] = acc[bm][bn][i];
    }
    __syncthreads();
    if (wave < 4) {
#pragma unroll
      for (int bm = 0; bm < NWM; ++bm) {
#pragma unroll
        for (int bn = 0; bn < NWN; ++bn) {
          const int j = n0 + col0 + 32 * bn + (lane & 31);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int lr0 = m0 + acc_row(row0, bm, 4 * g, lane);  // rows lr0 .. lr0 + 3
            if (lr0 >= Rp) continue;
            float va[4], vu[4], vp[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int lr = lr0 + q, i = 4 * g + q;
              va[q] = vu[q] = vp[q] = 0.f;
              if (lr < R) {
                const TT hb = hs[(lr - m0) * UD_BN + (j - n0)];
                if (active_bits(hb)) {
                  const float h = to_f32(hb), u = acc[bm][bn][i], da = xch[((bm * NWN + bn) * 16 + i) * 64];
                  va[q] = h * u;
                  vu[q] = da * h;
                  vp[q] = fmaf(da, u, lam);
                }
                du_rm[(size_t)lr * F + j] = from_f32<D>(vu[q]);
                dp_rm[(size_t)lr * F + j] = from_f32<D>(vp[q]);
              }
            }
            store_t4<D>(at + (size_t)j * as_stride, lr0, Rp, va);
            store_t4<D>(dut + (size_t)j * as_stride, lr0, Rp, vu);
            store_t4<D>(dpt + (size_t)j * as_stride, lr0, Rp, vp);
          }
        }
      }
    }
    __syncthreads();  // the hand-over area is the next tile's ring
  }
}

// ---------------------------------------------------------------------------
// dx of the dense rows: 256 x 128 tiles over K = 2F in two segments, du with
// W_u, then dpre with W_g.  When the row tiles are too few to fill the grid,
// K is cut into S ranges (a range may span the segment boundary) whose fp32
// partial tiles a reduction kernel adds in K order.

constexpr int BDX_BN = 128;
constexpr int BDX_WGS = 256;
constexpr int BDX_PARTIAL_TILES_MAX = 128;  // in 256 x 256 fp32 tiles (32 MB)

__host__ __device__ inline int bwd_dx_split(int tiles, int nk, int part_tiles) {
  return fallback_split(tiles, nk, DOWN_SPLIT_MAX, part_tiles * (256 / BDX_BN));
}

template <Dt D>
__device__ __forceinline__ void bwd_dx_tile(int tm, int tn, int k0, int k1, float *__restrict__ part,
                                            const typename DtT<D>::T *__restrict__ du_rm,
                                            const typename DtT<D>::T *__restrict__ dp_rm,
                                            const typename DtT<D>::T *__restrict__ wu,
                                            const typename DtT<D>::T *__restrict__ wg, int R, int F, int d,
                                            const int *__restrict__ dense_rows, int T,
                                            typename DtT<D>::T *__restrict__ dx) {
  using TT = typename DtT<D>::T;
  using K = BwdK<D>;
  constexpr int NB = BDX_BN / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int m0 = tm * GEMM_BM, n0 = tn * BDX_BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nks = F / K::KC;  // chunks per segment
  f32x16_t acc[2][NB];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < NB; ++bn) acc[bm][bn] = f32x16_t{};
  for (int seg = 0; seg < 2; ++seg) {
    const int b = max(k0, seg * nks), e = min(k1, (seg + 1) * nks);
    if (b >= e) continue;
    const int kb = b - seg * nks;
    const TT *A = seg ? dp_rm : du_rm;
    const TT *B = seg ? wg : wu;
    KRowLoader<GEMM_BM> la;
    la.init(tid, [&](int r) {
      return reinterpret_cast<const char *>(A) + (size_t)min(m0 + r, R - 1) * F * sizeof(TT) +
             (size_t)kb * KCHUNK_BYTES;
    });
    NColLoader<D, BDX_BN> lb;
    lb.init(tid, reinterpret_cast<const char *>(B) + (size_t)kb * K::KC * d * sizeof(TT), (size_t)d * sizeof(TT),
            n0);
    gemm_mainloop<D, BDX_BN>(acc, la, lb, e - b, smem);
  }
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
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int lr = m0 + acc_row(64 * wave, bm, i, lane);
      if (lr >= R) continue;
      const size_t prow = (size_t)min(max(dense_rows[lr], 0), T - 1);
#pragma unroll
      for (int bn = 0; bn < NB; ++bn) dx[prow * d + n0 + 32 * bn + col] = from_f32<D>(acc[bm][bn][i]);
    }
  }
}

template <Dt D>
__global__ __launch_bounds__(GEMM_THREADS) void k_bwd_dx(const typename DtT<D>::T *__restrict__ du_rm,
                                                        const typename DtT<D>::T *__restrict__ dp_rm,
                                                        const typename DtT<D>::T *__restrict__ wu,
                                                        const typename DtT<D>::T *__restrict__ wg,
                                                        const int *__restrict__ dense_rows,
                                                        const int *__restrict__ n_dense, int dense_cap, int T, int d,
                                                        int F, float *__restrict__ part, int part_tiles,
                                                        typename DtT<D>::T *__restrict__ dx) {
  const int R = dense_count(n_dense, dense_cap);
  const int ntl = d / BDX_BN;
  const int tiles = (R + GEMM_BM - 1) / GEMM_BM * ntl;
  const int nk = 2 * (F / BwdK<D>::KC);
  const int S = bwd_dx_split(tiles, nk, part_tiles);
  for (int w = blockIdx.x; w < tiles * S; w += gridDim.x) {
    const int tile = w / S, kc = w - tile * S;
    bwd_dx_tile<D>(tile / ntl, tile % ntl, kc * nk / S, (kc + 1) * nk / S,
                   S > 1 ? part + (size_t)w * GEMM_BM * BDX_BN : nullptr, du_rm, dp_rm, wu, wg, R, F, d, dense_rows,
                   T, dx);
  }
}

template <Dt D>
__global__ __launch_bounds__(256) void k_bwd_dx_reduce(const float *__restrict__ part,
                                                       const int *__restrict__ dense_rows,
                                                       const int *__restrict__ n_dense, int dense_cap, int T, int d,
                                                       int F, int part_tiles, typename DtT<D>::T *__restrict__ dx) {
  constexpr int PT = GEMM_BM * BDX_BN;
  const int R = dense_count(n_dense, dense_cap);
  const int ntl = d / BDX_BN;
  const int tiles = (R + GEMM_BM - 1) / GEMM_BM * ntl;
  const int nk = 2 * (F / BwdK<D>::KC);
  const int S = bwd_dx_split(tiles, nk, part_tiles);
  if (S == 1) return;
  const size_t total = (size_t)tiles * PT;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const int tile = (int)(e / PT);
    const int rem = (int)(e - (size_t)tile * PT);
    const int r = rem / BDX_BN, c = rem % BDX_BN;
    const int lr = (tile / ntl) * GEMM_BM + r;
    if (lr >= R) continue;
    const float *p = part + (size_t)tile * S * PT + down_part_index<BDX_BN>(r, c);
    float v = 0.f;
    for (int kc = 0; kc < S; ++kc) v += p[(size_t)kc * PT];
    const size_t prow = (size_t)min(max(dense_rows[lr], 0), T - 1);
    dx[prow * d + (size_t)(tile % ntl) * BDX_BN + c] = from_f32<D>(v);
  }
}

// ---------------------------------------------------------------------------
// Weight gradients of the dense rows: three matmuls of M = F units, N = d
// columns, K = NS * Rp over the transposed operands and the gathered rows,
// written to the gradients (the entry kernels add the other rows' part
// afterwards).  256 x 256 tiles.

template <Dt D>
__global__ __launch_bounds__(GEMM_THREADS) void k_bwd_dw(const typename DtT<D>::T *__restrict__ at,
                                                        const typename DtT<D>::T *__restrict__ dut,
                                                        const typename DtT<D>::T *__restrict__ dpt,
                                                        const typename DtT<D>::T *__restrict__ xr,
                                                        const typename DtT<D>::T *__restrict__ dyr,
                                                        const int *__restrict__ n_dense, int dense_cap, int F, int d,
                                                        int as_stride, float *__restrict__ dwg,
                                                        float *__restrict__ dwu, float *__restrict__ dwd) {
  using TT = typename DtT<D>::T;
  using K = BwdK<D>;
  constexpr int BN = 256, NB = BN / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int R = dense_count(n_dense, dense_cap);
  if (R == 0) return;
  const int nk = K::NS * pad_to(R, K::KC) / K::KC;
  const int mt = (F + GEMM_BM - 1) / GEMM_BM, ntl = d / BN, tiles = mt * ntl;
  const int prod = blockIdx.x / tiles;
  int tm, tn;
  tile_coords(blockIdx.x - prod * tiles, mt, ntl, tm, tn);
  const TT *A = prod == 0 ? dpt : prod == 1 ? dut : at;
  const TT *B = prod == 2 ? dyr : xr;
  float *out = prod == 0 ? dwg : prod == 1 ? dwu : dwd;
  const int m0 = tm * GEMM_BM, n0 = tn * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  KRowLoader<GEMM_BM> la;
  la.init(tid, [&](int r) {
    return reinterpret_cast<const char *>(A) + (size_t)min(m0 + r, F - 1) * as_stride * sizeof(TT);
  });
  NColLoader<D, BN> lb;
  lb.init(tid, B, (size_t)d * sizeof(TT), n0);
  f32x16_t acc[2][NB];
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < NB; ++bn) acc[bm][bn] = f32x16_t{};
  gemm_mainloop<D, BN>(acc, la, lb, nk, smem);
  const int col = lane & 31;
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int lr = m0 + acc_row(64 * wave, bm, i, lane);
      if (lr >= F) continue;
      float *o = out + (size_t)lr * d + n0 + col;
#pragma unroll
      for (int bn = 0; bn < NB; ++bn) o[32 * bn] = acc[bm][bn][i];
    }
  }
}

// ---------------------------------------------------------------------------

// Capacity of the dx split's partial area in 256 x 256 fp32 tiles, and the
// padded row count of the gathered and transposed operands.
int backward_dense_partial_tiles(int dense_cap, int d) {
  if (dense_cap <= 0) return 0;
  // a split gives at most BDX_WGS work items, whatever the row count
  const int tiles = (dense_cap + GEMM_BM - 1) / GEMM_BM * (d / BDX_BN);
  const int items = std::min(BDX_WGS, tiles * DOWN_SPLIT_MAX);
  return std::min(BDX_PARTIAL_TILES_MAX, (items * GEMM_BM * BDX_BN + FALLBACK_SPLIT_TILE - 1) / FALLBACK_SPLIT_TILE);
}

int backward_dense_rows_padded(int dense_cap, Dt dt) {
  return pad_to(dense_cap, dt == Dt::BF16 ? BwdK<Dt::BF16>::KC : BwdK<Dt::F32>::KC);
}

template <Dt D>
static hipError_t launch_dense_dx(const BackwardArgs &a, hipStream_t st) {
  using TT = typename DtT<D>::T;
  using K = BwdK<D>;
  hipError_t e;
  const int rcp = pad_to(a.dense_cap, K::KC), as_stride = K::NS * rcp;
  // grids of at most one workgroup per CU for the gather and U/DA kernels,
  // which loop (when no row is dense they only read the count and exit); the
  // reduction keeps 1024 workgroups, which it needs to hide its load latency
  hipLaunchKernelGGL(k_bwd_gather<D>, dim3(std::min(K::NS * rcp, 256)), dim3(256), 0, st, (const TT *)a.x,
                     (const TT *)a.dy, a.dense_rows, a.n_dense, a.dense_cap, a.T, a.d, (TT *)a.bd_xr,
                     (TT *)a.bd_dyr);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const int ud_lds = gemm_dma_lds_bytes<DiagCfg>(256);
  if ((e = hipFuncSetAttribute((const void *)k_bwd_ud<D>, hipFuncAttributeMaxDynamicSharedMemorySize, ud_lds)) !=
      hipSuccess)
    return e;
  const int ud_items = (a.dense_cap + UD_BM - 1) / UD_BM * (a.F / UD_BN);
  hipLaunchKernelGGL(k_bwd_ud<D>, dim3(std::min(ud_items, 256)), dim3(DiagCfg::THREADS), ud_lds, st,
                     (const TT *)a.x, (const TT *)a.dy, (const TT *)a.wu, (const TT *)a.wd, a.dense_rows, a.n_dense,
                     a.dense_cap, (const TT *)a.dense, a.T, a.d, a.F, a.lam, (TT *)a.bd_du, (TT *)a.bd_dp,
                     (TT *)a.bd_at, (TT *)a.bd_dut, (TT *)a.bd_dpt, as_stride);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const int dx_lds = gemm_lds_bytes(BDX_BN);
  if ((e = hipFuncSetAttribute((const void *)k_bwd_dx<D>, hipFuncAttributeMaxDynamicSharedMemorySize, dx_lds)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL(k_bwd_dx<D>, dim3(BDX_WGS), dim3(GEMM_THREADS), dx_lds, st, (const TT *)a.bd_du,
                     (const TT *)a.bd_dp, (const TT *)a.wu, (const TT *)a.wg, a.dense_rows, a.n_dense, a.dense_cap,
                     a.T, a.d, a.F, a.bd_part, a.bd_part_tiles, (TT *)a.dx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.bd_part_tiles >= 1) {
    hipLaunchKernelGGL(k_bwd_dx_reduce<D>, dim3(1024), dim3(256), 0, st, (const float *)a.bd_part, a.dense_rows,
                       a.n_dense, a.dense_cap, a.T, a.d, a.F, a.bd_part_tiles, (TT *)a.dx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <Dt D>
static hipError_t launch_dense_dw(const BackwardArgs &a, hipStream_t st) {
  using TT = typename DtT<D>::T;
  using K = BwdK<D>;
  hipError_t e;
  const int as_stride = K::NS * pad_to(a.dense_cap, K::KC);
  const int dw_lds = gemm_lds_bytes(256);
  if ((e = hipFuncSetAttribute((const void *)k_bwd_dw<D>, hipFuncAttributeMaxDynamicSharedMemorySize, dw_lds)) !=
      hipSuccess)
    return e;
  const int dw_tiles = (a.F + GEMM_BM - 1) / GEMM_BM * (a.d / 256);
  hipLaunchKernelGGL(k_bwd_dw<D>, dim3(3 * dw_tiles), dim3(GEMM_THREADS), dw_lds, st, (const TT *)a.bd_at,
                     (const TT *)a.bd_dut, (const TT *)a.bd_dpt, (const TT *)a.bd_xr, (const TT *)a.bd_dyr,
                     a.n_dense, a.dense_cap, a.F, a.d, as_stride, a.dwg, a.dwu, a.dwd);
  return hipGetLastError();
}

hipError_t ffn_backward_dense_dx(const BackwardArgs &a, hipStream_t s) {
  if (a.T <= 0 || a.dense_cap <= 0) return hipSuccess;
  return a.dtype == Dt::BF16 ? launch_dense_dx<Dt::BF16>(a, s) : launch_dense_dx<Dt::F32>(a, s);
}

hipError_t ffn_backward_dense_dw(const BackwardArgs &a, hipStream_t s) {
  if (a.T <= 0 || a.dense_cap <= 0) return hipSuccess;
  return a.dtype == Dt::BF16 ? launch_dense_dw<Dt::BF16>(a, s) : launch_dense_dw<Dt::F32>(a, s);
}

}  // namespace twell
