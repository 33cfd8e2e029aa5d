// TwELL -> hybrid conversion (the training format of gist.science "Sparser,
// Faster, Lighter Transformer Language Models", Resumen Técnico §2.A: rows
// with few non-zeros in a compact ELL matrix, the others in a dense backup;
// the conversion kernel is one of the training kernels of §2.B).
//
//   k_hybrid_rows:  one wave per row.  The row's TwELL counts give its true
//                   entry count and whether it overflowed TwELL.  A row with
//                   at most `width` entries becomes an ELL row: from its
//                   TwELL slots (with at most 64 tiles one lane per ELL
//                   position, its tile found by a search over the tiles'
//                   prefix counts; otherwise one lane per tile), or, when it
//                   overflowed TwELL, by a ballot compaction of its dense
//                   backup row.  Other rows get
//                   all-padding ELL slots.  With saved u, an ELL row from
//                   TwELL slots copies the slots' u too; one from the dense
//                   backup marks its u as not saved (NaN in its first slot).
//   k_compact_gt:   ascending list of the rows with more than `width` entries.
//   k_hybrid_dense: one workgroup per listed row: the dense backup row, copied
//                   from TwELL's dense backup or scattered from the slots.
#include "gather.hpp"
#include "launch.hpp"

#include <algorithm>

namespace twell {

constexpr int HY_WAVES = 4;

template <Dt D>
__global__ __launch_bounds__(64 * HY_WAVES) void k_hybrid_rows(
    const uint16_t *__restrict__ cnt, const typename DtT<D>::T *__restrict__ val, const uint8_t *__restrict__ idx,
    const int *__restrict__ ovf_rows, const int *__restrict__ n_ovf, int ovf_cap,
    const typename DtT<D>::T *__restrict__ tw_dense, int T, int F, int tile, int cap, int width,
    int *__restrict__ out_cnt, typename DtT<D>::T *__restrict__ out_val, int *__restrict__ out_col,
    const float *__restrict__ tw_u, float *__restrict__ out_u) {
  using TT = typename DtT<D>::T;
  __shared__ int tile_incl[HY_WAVES][64];  // inclusive entry counts over a row's tiles
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * HY_WAVES + wave;
  if (t >= T) return;
  const int nt = F / tile;
  const uint16_t *crow = cnt + (size_t)t * nt;
  int total = 0;
  bool over = false;
  for (int kb = 0; kb < nt; kb += 64) {
    const int k = kb + lane;
    const int c = k < nt ? (int)crow[k] : 0;
    total += c;
    over |= c > cap;
  }
  total = __builtin_amdgcn_readlane(wave_incl_scan(total), 63);
  const bool tw_ovf = ballot(over) != 0;
  if (lane == 0) out_cnt[t] = total;
  TT *vrow = out_val + (size_t)t * width;
  int *crow_out = out_col + (size_t)t * width;
  const int n_ell = total <= width ? total : 0;  // ELL entries written below
  if (total <= width) {
    if (!tw_ovf && nt <= 64) {
      // one lane per output position e < total: its tile is the first whose
      // inclusive count exceeds e (a search over the row's tile counts in
      // LDS), its slot e minus the entries of the tiles before
      const int n = lane < nt ? (int)crow[lane] : 0;
      int *inc = tile_incl[wave];
      inc[lane] = wave_incl_scan(n);
      wave_sync_lds();
      for (int e = lane; e < total; e += 64) {
        int lo = 0, hi = nt - 1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (inc[mid] > e)
            hi = mid;
          else
            lo = mid + 1;
        }
        const int s = e - (lo > 0 ? inc[lo - 1] : 0);
        const size_t slot = ((size_t)t * nt + lo) * cap + s;
        vrow[e] = val[slot];
        crow_out[e] = lo * tile + (idx[slot] & (tile - 1));
        if (out_u != nullptr) out_u[(size_t)t * width + e] = tw_u[slot];
      }
    } else if (!tw_ovf) {
      // lanes take tiles (64 at a time); a lane copies its tile's entries to
      // the row position given by a prefix count over the tiles
      int before = 0;  // entries of the tiles before the chunk
      for (int kb = 0; kb < nt; kb += 64) {
        const int k = kb + lane;
        const int n = k < nt ? (int)crow[k] : 0;
        const int incl = wave_incl_scan(n);
        const int pos0 = before + incl - n;
        const size_t slot0 = ((size_t)t * nt + k) * cap;
        for (int s = 0; s < n; ++s) {
          if (pos0 + s < width) {
            vrow[pos0 + s] = val[slot0 + s];
            crow_out[pos0 + s] = k * tile + (idx[slot0 + s] & (tile - 1));
            if (out_u != nullptr) out_u[(size_t)t * width + pos0 + s] = tw_u[slot0 + s];
          }
        }
        before += __builtin_amdgcn_readlane(incl, 63);
      }
    } else {
      // the TwELL slots lost entries of this row: compact its dense backup row
      // (its u was not saved)
      if (out_u != nullptr && lane == 0) out_u[(size_t)t * width] = __builtin_nanf("");
      const int r = find_row(ovf_rows, min(*n_ovf, ovf_cap), t);
      const TT *drow = tw_dense + (size_t)max(r, 0) * F;
      int before = 0;
      for (int jb = 0; r >= 0 && jb < F; jb += 64) {
        const int j = jb + lane;
        const TT v = j < F ? drow[j] : TT(0);
        const bool act = j < F && active_bits(v);
        const uint64_t m = ballot(act);
        const int pos = before + mbcnt(m);
        if (act && pos < width) {
          vrow[pos] = v;
          crow_out[pos] = j;
        }
        before += popc64(m);
      }
    }
  }
  // padding: +0 values, column 0
  for (int s = n_ell + lane; s < width; s += 64) {
    vrow[s] = TT(0);
    crow_out[s] = 0;
  }
}

// Ascending list of the rows t with cnt[t] > width; one workgroup.
constexpr int HY_COMPACT_THREADS = 1024;
__global__ __launch_bounds__(HY_COMPACT_THREADS) void k_compact_gt(const int *__restrict__ cnt, int T, int width,
                                                                    int *__restrict__ rows, int rows_cap,
                                                                    int *__restrict__ n_rows) {
  __shared__ int wcount[HY_COMPACT_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < T; base += HY_COMPACT_THREADS) {
    const int t = base + tid;
    const bool f = t < T && cnt[t] > width;
    const uint64_t m = ballot(f);
    if (lane == 0) wcount[wave] = popc64(m);
    __syncthreads();
    int before = carry, total = 0;
    for (int w = 0; w < HY_COMPACT_THREADS / 64; ++w) {
      before += (w < wave) ? wcount[w] : 0;
      total += wcount[w];
    }
    if (f) {
      const int pos = before + mbcnt(m);
      if (pos < rows_cap) rows[pos] = t;
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) *n_rows = carry;
}

constexpr int HY_DENSE_THREADS = 256;

template <Dt D>
__global__ __launch_bounds__(HY_DENSE_THREADS) void k_hybrid_dense(
    const uint16_t *__restrict__ cnt, const typename DtT<D>::T *__restrict__ val, const uint8_t *__restrict__ idx,
    const int *__restrict__ ovf_rows, const int *__restrict__ n_ovf, int ovf_cap,
    const typename DtT<D>::T *__restrict__ tw_dense, int F, int tile, int cap, const int *__restrict__ dense_rows,
    const int *__restrict__ n_dense, int dense_cap, typename DtT<D>::T *__restrict__ out_dense) {
  using TT = typename DtT<D>::T;
  const int n = min(*n_dense, dense_cap);
  const int nt = F / tile;
  for (int r = blockIdx.x; r < n; r += gridDim.x) {
    const int t = dense_rows[r];
    TT *orow = out_dense + (size_t)r * F;
    const int p = find_row(ovf_rows, min(*n_ovf, ovf_cap), t);
    if (p >= 0) {
      const TT *drow = tw_dense + (size_t)p * F;
      for (int j = threadIdx.x; j < F; j += HY_DENSE_THREADS) orow[j] = drow[j];
    } else {
      for (int j = threadIdx.x; j < F; j += HY_DENSE_THREADS) orow[j] = TT(0);
      __syncthreads();
      // every entry of a row that did not overflow TwELL is in its slots
      for (int q = threadIdx.x; q < nt * cap; q += HY_DENSE_THREADS) {
        const int k = q / cap, s = q - k * cap;
        const size_t slot = ((size_t)t * nt + k) * cap + s;
        const int c = idx[slot] & (tile - 1);  // an index is taken modulo the tile width
        if (s < (int)cnt[(size_t)t * nt + k]) orow[k * tile + c] = val[slot];
      }
    }
    __syncthreads();
  }
}

template <Dt D>
static hipError_t launch_hybrid(const HybridArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  hipLaunchKernelGGL(k_hybrid_rows<D>, dim3((a.T + HY_WAVES - 1) / HY_WAVES), dim3(64 * HY_WAVES), 0, s, a.cnt,
                     (const TT *)a.val, a.idx, a.ovf_rows, a.n_ovf, a.ovf_cap, (const TT *)a.tw_dense, a.T, a.F,
                     a.tile, a.cap, a.width, a.out_cnt, (TT *)a.out_val, a.out_col, a.tw_u, a.out_u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_compact_gt, dim3(1), dim3(HY_COMPACT_THREADS), 0, s, a.out_cnt, a.T, a.width, a.dense_rows,
                     a.dense_cap, a.n_dense);
  e = hipGetLastError();
  if (e != hipSuccess || a.out_dense == nullptr || a.dense_cap == 0) return e;
  const int grid = std::min(a.T, 256);
  hipLaunchKernelGGL(k_hybrid_dense<D>, dim3(grid), dim3(HY_DENSE_THREADS), 0, s, a.cnt, (const TT *)a.val, a.idx,
                     a.ovf_rows, a.n_ovf, a.ovf_cap, (const TT *)a.tw_dense, a.F, a.tile, a.cap, a.dense_rows,
                     a.n_dense, a.dense_cap, (TT *)a.out_dense);
  return hipGetLastError();
}

hipError_t twell_to_hybrid_launch(const HybridArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return a.dtype == Dt::BF16 ? launch_hybrid<Dt::BF16>(a, s) : launch_hybrid<Dt::F32>(a, s);
}

}  // namespace twell
