// Backward pass of the ReLU-gated FFN layer from its hybrid activations: the
// training kernels of gist.science "Sparser, Faster, Lighter Transformer
// Language Models", Resumen Técnico §2.B (hybrid-times-dense and
// dense-times-hybrid products, sparse transpose for the gradients), on the
// hybrid format of §2.A.  With u = x W_u^T, a = h * u, y = a W_d and the L1
// term lam * ||h||_1, for every active entry (t, j) of h:
//
//   da = dy_t . W_d[j],  du = da * h,  dpre = da * u + lam
//   dx_t    = sum_j du W_u[j] + dpre W_g[j]             (hybrid x dense)
//   dW_u[j] = sum_t du x_t,  dW_g[j] = sum_t dpre x_t,
//   dW_d[j] = sum_t a dy_t                               (transpose x dense)
//
// Kernels, in launch order:
//   k_bw_dense_cols   compacted column lists of the dense backup rows
//   k_bw_count        per block of 64 rows, a 64-bit row mask per column in
//                     LDS; writes the per-column entry counts of the block
//   k_bw_colscan      per column, the running count over the blocks
//   k_bw_colptr       column starts of the transposed (column-major) lists,
//                     and, when the dense rows are walked entry by entry,
//                     the order in which the per-row kernels take the rows:
//                     the long dense rows first
//   k_bw_pos          each entry's place in its column's list: rows in
//                     ascending order, from the same LDS row masks
//   k_bw_entries      per (row, group of hidden units): u and da by gathering
//                     W_u and W_d rows (the group's rows stay in one XCD's
//                     L2; W_d rows only where the forward saved u), then du,
//                     dpre and a; written per entry and, in column order, to
//                     the transposed lists
//   k_bw_dx           per (row, column slice of d): dx over the row's entries
//   k_bw_dw           per (hidden unit, column slice): dW_u and dW_g rows
//                     over the unit's transposed list (x rows), then in a
//                     second launch dW_d (dy rows)
// and, when the hidden size allows it (a multiple of 128), the dense backup
// rows on the matrix cores (bw_dense.hip) between k_bw_dx and k_bw_dw; their
// lists are empty here.  Otherwise k_bw_dense_cols lists their active columns
// first and they are walked like the others.
// Every sum runs in a fixed order (entry order of a row, ascending rows of a
// column), so the results are deterministic.  No atomics touch global memory.
#include "gather.hpp"
#include "launch.hpp"

#include <algorithm>

namespace twell {

constexpr int BW_THREADS = 256;
constexpr int BW_WAVES = BW_THREADS / 64;
// The row-mask kernels of the transpose walk a block's rows through dependent
// loads (count, then columns): 16 waves per workgroup, 4 rows each.
constexpr int TR_THREADS = 1024;
constexpr int TR_WAVES = TR_THREADS / 64;
constexpr int BW_RB = 64;     // rows per block of the transpose (one bit each)
constexpr int DX_SLICE = 128; // columns of d per dx slice
constexpr int DW_SLICE = 256; // columns of d per dW slice

template <class TT>
struct RowSrc {
  const int *cnt;         // [T] active entries per row
  const TT *val;          // [T][width]
  const int *col;         // [T][width]
  const int *dense_rows;  // ascending dense rows
  const int *n_dense;
  int dense_cap;
  const TT *dense;        // [dense_cap][F]
  const int *dcol;        // [dense_cap][F] compacted columns of the dense rows
  const int *dn;          // [dense_cap] their lengths
  int T, F, width;
  bool dense_mma;         // dense rows go to the matrix-core kernels: empty lists here
  const float *u;         // [T][width] saved u of the ELL slots (NaN in slot 0: not saved), or null
};

// The entry list of row t: the hybrid's ELL slots, or the compacted columns
// of its dense backup row (r >= 0).  Entry slots are numbered t * width + i
// for ELL rows and T * width + r * F + i for dense row r.  With dense_mma the
// dense rows' lists are empty (the matrix-core kernels take those rows).
struct RowList {
  const int *col;
  int n, r;
  size_t slot0;
};

template <class TT>
__device__ __forceinline__ RowList row_list(const RowSrc<TT> &s, int t) {
  RowList L;
  const int c = s.cnt[t];
  if (c <= s.width) {
    L.col = s.col + (size_t)t * s.width;
    L.n = max(c, 0);
    L.r = -1;
    L.slot0 = (size_t)t * s.width;
  } else if (s.dense_mma) {
    L.col = s.col;
    L.n = 0;
    L.r = -1;
    L.slot0 = 0;
  } else {
    const int r = find_row(s.dense_rows, min(*s.n_dense, s.dense_cap), t);
    L.r = r;
    L.col = s.dcol + (size_t)max(r, 0) * s.F;
    L.n = r >= 0 ? s.dn[r] : 0;
    L.slot0 = (size_t)s.T * s.width + (size_t)max(r, 0) * s.F;
  }
  return L;
}

// Columns come from the caller's hybrid matrix: keep every address in range.
__device__ __forceinline__ int clamp_col(int j, int F) { return (unsigned)j < (unsigned)F ? j : 0; }

// ---------------------------------------------------------------------------
// Compacted column lists of the dense backup rows: one wave per row, ballots
// over the row in column order.
template <Dt D>
__global__ __launch_bounds__(BW_THREADS) void k_bw_dense_cols(const typename DtT<D>::T *__restrict__ dense,
                                                             const int *__restrict__ n_dense, int dense_cap, int F,
                                                             int *__restrict__ dcol, int *__restrict__ dn) {
  const int lane = threadIdx.x & 63;
  const int nd = min(*n_dense, dense_cap);
  for (int r = blockIdx.x * BW_WAVES + (threadIdx.x >> 6); r < nd; r += gridDim.x * BW_WAVES) {
    const typename DtT<D>::T *row = dense + (size_t)r * F;
    int *out = dcol + (size_t)r * F;
    int before = 0;
    for (int jb = 0; jb < F; jb += 64) {
      const int j = jb + lane;
      const bool act = j < F && active_bits(row[j]);
      const uint64_t m = ballot(act);
      if (act) out[before + mbcnt(m)] = j;
      before += popc64(m);
    }
    if (lane == 0) dn[r] = before;
  }
}

// ---------------------------------------------------------------------------
// Transpose.  Block b covers rows [64 b, 64 b + 64); mask[j] has bit (t - 64 b)
// set when row t has an entry in column j.

template <class TT>
__device__ __forceinline__ void block_masks(const RowSrc<TT> &s, int b, unsigned long long *mask) {
  for (int j = threadIdx.x; j < s.F; j += TR_THREADS) mask[j] = 0ull;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t_end = min(s.T, (b + 1) * BW_RB);
  for (int t = b * BW_RB + (threadIdx.x >> 6); t < t_end; t += TR_WAVES) {
    const RowList L = row_list(s, t);
    const unsigned long long bit = 1ull << (t - b * BW_RB);
    for (int i = lane; i < L.n; i += 64) atomicOr(&mask[clamp_col(L.col[i], s.F)], bit);
  }
  __syncthreads();
}

template <class TT>
__global__ __launch_bounds__(TR_THREADS) void k_bw_count(RowSrc<TT> s, uint8_t *__restrict__ blk) {
  extern __shared__ unsigned long long mask[];
  block_masks(s, blockIdx.x, mask);
  uint8_t *out = blk + (size_t)blockIdx.x * s.F;
  for (int j = threadIdx.x; j < s.F; j += TR_THREADS) out[j] = (uint8_t)__popcll(mask[j]);
}

// boff[b][j] = entries of column j in blocks before b; tot[j] = all of them.
__global__ __launch_bounds__(BW_THREADS) void k_bw_colscan(const uint8_t *__restrict__ blk, int NB, int F,
                                                          int *__restrict__ boff, int *__restrict__ tot) {
  const int j = blockIdx.x * BW_THREADS + threadIdx.x;
  if (j >= F) return;
  int run = 0;
  int b = 0;
  for (; b + 8 <= NB; b += 8) {
    int c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) c[q] = blk[(size_t)(b + q) * F + j];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      boff[(size_t)(b + q) * F + j] = run;
      run += c[q];
    }
  }
  for (; b < NB; ++b) {
    boff[(size_t)b * F + j] = run;
    run += blk[(size_t)b * F + j];
  }
  tot[j] = run;
}

// colptr[j] = sum of tot[0..j), colptr[F] = the total; one workgroup, each
// thread a contiguous run of columns.
constexpr int COLPTR_THREADS = 1024;
template <class TT>
__device__ __forceinline__ void row_order(const RowSrc<TT> &s, int *__restrict__ order, int *wcount);

// With an order array, also writes the row order of the per-row kernels
// (row_order, below).
template <class TT>
__global__ __launch_bounds__(COLPTR_THREADS) void k_bw_colptr(const int *__restrict__ tot, int F,
                                                             int *__restrict__ colptr, RowSrc<TT> s,
                                                             int *__restrict__ order) {
  __shared__ int wsum[COLPTR_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int PER_MAX = 16;  // F <= 16384
  const int per = (F + COLPTR_THREADS - 1) / COLPTR_THREADS;
  const int j0 = min(F, tid * per), j1 = min(F, j0 + per);
  int v[PER_MAX];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < PER_MAX; ++q) {
    v[q] = j0 + q < j1 ? tot[j0 + q] : 0;
    mine += v[q];
  }
  const int incl = wave_incl_scan(mine);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = incl - mine;
  for (int w = 0; w < wave; ++w) before += wsum[w];
#pragma unroll
  for (int q = 0; q < PER_MAX; ++q) {
    if (j0 + q < j1) colptr[j0 + q] = before;
    before += v[q];
  }
  if (tid == COLPTR_THREADS - 1) colptr[F] = before;
  if (order != nullptr) {
    __syncthreads();
    row_order(s, order, wsum);
  }
}

// The order in which the per-row kernels take the rows: the stored dense rows
// first (their lists are ~F * density long, the others ~width or less), then
// every other row in ascending order, so that the long rows start early
// instead of finishing last.  One workgroup; order[0..T) is a permutation.
// (Runs in the column-starts kernel: one workgroup of COLPTR_THREADS.)
template <class TT>
__device__ __forceinline__ void row_order(const RowSrc<TT> &s, int *__restrict__ order, int *wcount) {
  constexpr int ORDER_THREADS = COLPTR_THREADS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nd = max(min(*s.n_dense, s.dense_cap), 0);
  for (int i = tid; i < min(nd, s.T); i += ORDER_THREADS) order[i] = s.dense_rows[i];
  constexpr int PER = 8;  // consecutive rows per thread per round
  int carry = nd;
  for (int base = 0; base < s.T; base += ORDER_THREADS * PER) {
    const int t0 = base + tid * PER;
    int c[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) c[q] = t0 + q < s.T ? s.cnt[t0 + q] : 0;
    bool rest[PER];
    int n = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      rest[q] = t0 + q < s.T && (c[q] <= s.width || find_row(s.dense_rows, nd, t0 + q) < 0);
      n += rest[q];
    }
    const int incl = wave_incl_scan(n);
    if (lane == 63) wcount[wave] = incl;
    __syncthreads();
    int pos = carry + incl - n, total = 0;
    for (int w = 0; w < ORDER_THREADS / 64; ++w) {
      pos += (w < wave) ? wcount[w] : 0;
      total += wcount[w];
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (rest[q]) {
        if (pos < s.T) order[pos] = t0 + q;
        ++pos;
      }
    }
    carry += total;
    __syncthreads();
  }
}

// pos[slot] = colptr[j] + boff[b][j] + (rows of the block before t with an
// entry in column j).
template <class TT>
__global__ __launch_bounds__(TR_THREADS) void k_bw_pos(RowSrc<TT> s, const int *__restrict__ colptr,
                                                      const int *__restrict__ boff, int *__restrict__ pos) {
  extern __shared__ unsigned long long mask[];
  const int b = blockIdx.x;
  block_masks(s, b, mask);
  const int lane = threadIdx.x & 63;
  const int t_end = min(s.T, (b + 1) * BW_RB);
  const int *bo = boff + (size_t)b * s.F;
  for (int t = b * BW_RB + (threadIdx.x >> 6); t < t_end; t += TR_WAVES) {
    const RowList L = row_list(s, t);
    const unsigned long long below = (1ull << (t - b * BW_RB)) - 1ull;
    for (int i = lane; i < L.n; i += 64) {
      const int j = clamp_col(L.col[i], s.F);
      pos[L.slot0 + i] = colptr[j] + bo[j] + __popcll(mask[j] & below);
    }
  }
}

// ---------------------------------------------------------------------------
// Entry gradients.

// First index i in [0, n) with c[i] >= key (c ascending), for the whole wave:
// 64 samples per round narrow the range until one load per lane settles it.
__device__ __forceinline__ int wave_lower_bound(const int *__restrict__ c, int n, int key) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;  // the answer lies in [lo, hi]
  while (hi - lo > 64) {
    const int step = (hi - lo + 63) / 64;
    const int p = lo + lane * step;
    const int k = popc64(ballot(p < hi && c[p] < key));  // samples below the key
    if (k == 0) return lo;
    const int nlo = lo + (k - 1) * step + 1;
    hi = min(lo + k * step, hi);
    lo = nlo;
  }
  const int p = lo + lane;
  return lo + popc64(ballot(p < hi && c[p] < key));
}

// One wave per (row t, group of hidden units), groups placed on XCDs as in
// the forward's up projection.  x_t and dy_t stay in registers (NC 16-byte
// chunks per lane each); U entries are in flight, each a W_u row and a W_d
// row.  The 2U dot products are reduced together: after Reduce<2U> the lanes
// of one 16-lane row (U = 2) or half-wave (U = 1) hold u of an entry and
// their partner rows hold its da.
template <Dt D, int NC, int U>
__global__ __launch_bounds__(SP_THREADS) void k_bw_entries(RowSrc<typename DtT<D>::T> s,
                                                          const typename DtT<D>::T *__restrict__ x,
                                                          const typename DtT<D>::T *__restrict__ dy,
                                                          const typename DtT<D>::T *__restrict__ wu,
                                                          const typename DtT<D>::T *__restrict__ wd, float lam,
                                                          int d, int upg, int n_groups, int tok_per_wg, int n_tb,
                                                          const int *__restrict__ pos, f32x2_t *__restrict__ ent,
                                                          u32x4_t *__restrict__ csc,
                                                          const int *__restrict__ order) {
  using TT = typename DtT<D>::T;
  static_assert(U == 1 || U == 2, "one or two entries in flight");
  constexpr int EPC = 16 / sizeof(TT);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int g, tb;
  group_coords(blockIdx.x, n_groups, n_tb, g, tb);
  if (g >= n_groups) return;
  const int j0 = g * upg, j1 = min(s.F, j0 + upg);
  const size_t w_bytes = (size_t)s.F * d * sizeof(TT);
  const __amdgpu_buffer_rsrc_t wur = buffer_rsrc(wu, w_bytes), wdr = buffer_rsrc(wd, w_bytes);
  const uint32_t lane_off = lane * 16;
  const uint32_t row_bytes = (uint32_t)d * sizeof(TT);
  const int my = U == 2 ? lane >> 5 : 0;  // the entry whose u this lane's row holds (storer lanes)
  const bool storer = U == 2 ? (lane & 31) == 0 : lane == 0;
  const int partner = U == 2 ? 16 : 32;
  __shared__ f32x2_t stage_e[SP_WAVES][64];
  f32x2_t *S = stage_e[wave];

  // the workgroup's rows, one per lane (tok_per_wg <= 64), read once
  const int r_i = min(tb * tok_per_wg + min(lane, tok_per_wg - 1), s.T - 1);
  const int my_row = order != nullptr ? order[r_i] : r_i;
  for (int it = wave; it < tok_per_wg; it += SP_WAVES) {
    const int ti = tb * tok_per_wg + it;
    if (ti >= s.T) break;
    const int t = min(max(__builtin_amdgcn_readlane(my_row, it), 0), s.T - 1);  // a valid hybrid gives a permutation
    const RowList L = row_list(s, t);
    if (L.n == 0) continue;
    // the row's entries in [j0, j1): its (ascending) columns below j0 and j1
    // counted in one pass of independent loads for an ELL-sized row, a
    // search otherwise
    int eb, ee;
    if (L.n <= 256) {
      int cb = 0, ce = 0;
#pragma unroll
      for (int k = 0; k < 256; k += 64) {
        if (k < L.n) {
          const int p = k + lane;
          const int c = p < L.n ? L.col[p] : 0x7FFFFFFF;
          cb += popc64(ballot(c < j0));
          ce += popc64(ballot(c < j1));
        }
      }
      eb = cb;
      ee = ce;
    } else {
      eb = wave_lower_bound(L.col, L.n, j0);
      ee = wave_lower_bound(L.col, L.n, j1);
    }
    if (eb >= ee) continue;
    // the row's u saved by the forward (an ELL row whose first slot holds a
    // number): x_t is not needed and only the W_d rows are gathered
    const bool saved = s.u != nullptr && L.r < 0 && !__builtin_isnan(s.u[(size_t)t * s.width]);
    const TT *xt = x + (size_t)t * d;
    const TT *dyt = dy + (size_t)t * d;
    u32x4_t xr[NC], gr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) gr[c] = *reinterpret_cast<const u32x4_t *>(dyt + (c * 64 + lane) * EPC);
    if (!saved) {
#pragma unroll
      for (int c = 0; c < NC; ++c) xr[c] = *reinterpret_cast<const u32x4_t *>(xt + (c * 64 + lane) * EPC);
    }
    for (int e0 = eb; e0 < ee; e0 += 64) {
      const int ne = min(64, ee - e0);
      // the lane's entry of this chunk (the last one repeated past the end)
      const int i = e0 + min(lane, ne - 1);
      const int j = clamp_col(L.col[i], s.F);
      const uint32_t moff = (uint32_t)j * row_bytes;
      const float hv = L.r < 0 ? to_f32(s.val[(size_t)t * s.width + i]) : to_f32(s.dense[(size_t)L.r * s.F + j]);
      const int pv = pos[L.slot0 + i];
      const float uv = saved ? s.u[(size_t)t * s.width + i] : 0.f;
      // Each entry's u (recomputed rows) and da go to the wave's LDS stage;
      // the entry's own lane then forms du, dpre and a and writes them, one
      // store instruction per 64 entries for each output.
      if (saved) {
        for (int u0 = 0; u0 < ne; u0 += U) {
          u32x4_t b[U][NC];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint32_t off = read_lane(moff, min(u0 + u, ne - 1));
            if (u0 + u < ne) {
#pragma unroll
              for (int c = 0; c < NC; ++c) b[u][c] = buffer_load<u32x4_t>(wdr, lane_off + c * 1024, off);
            } else {
#pragma unroll
              for (int c = 0; c < NC; ++c) b[u][c] = u32x4_t{0u, 0u, 0u, 0u};
            }
          }
          float p[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            p[u] = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) p[u] = dot16(gr[c], b[u][c], p[u], TT());
          }
          // after Reduce<U> the storer lanes hold da of their entry
          const float da = Reduce<U>::run(p);
          if (storer && u0 + my < ne) S[u0 + my] = f32x2_t{0.f, da};
        }
      } else {
        for (int u0 = 0; u0 < ne; u0 += U) {
          u32x4_t a[U][NC], b[U][NC];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint32_t off = read_lane(moff, min(u0 + u, ne - 1));
            if (u0 + u < ne) {
#pragma unroll
              for (int c = 0; c < NC; ++c) {
                a[u][c] = buffer_load<u32x4_t>(wur, lane_off + c * 1024, off);
                b[u][c] = buffer_load<u32x4_t>(wdr, lane_off + c * 1024, off);
              }
            } else {
#pragma unroll
              for (int c = 0; c < NC; ++c) a[u][c] = b[u][c] = u32x4_t{0u, 0u, 0u, 0u};
            }
          }
          float p[2 * U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            p[u] = 0.f;
            p[U + u] = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              p[u] = dot16(xr[c], a[u][c], p[u], TT());
              p[U + u] = dot16(gr[c], b[u][c], p[U + u], TT());
            }
          }
          const float tot = Reduce<2 * U>::run(p);
          const float other = __shfl_xor(tot, partner, 64);
          if (storer && u0 + my < ne) S[u0 + my] = f32x2_t{tot, other};  // u, da
        }
      }
      wave_sync_lds();
      if (lane < ne) {
        const f32x2_t q = S[lane];
        const float uu = saved ? uv : q[0], da = q[1];
        const float du = da * hv, dp = fmaf(da, uu, lam), av = hv * uu;
        ent[L.slot0 + i] = f32x2_t{du, dp};
        csc[pv] = u32x4_t{(uint32_t)t, __float_as_uint(av), __float_as_uint(du), __float_as_uint(dp)};
      }
      wave_sync_lds();
    }
  }
}

// ---------------------------------------------------------------------------
// dx and dW: one wave per (row or unit, column slice of d), slice s
// on XCD s % 8.  Each lane loads 16 bytes per instruction, LPE lanes per
// entry, EPI entries per instruction; the list goes through LDS 64 entries at
// a time; the EPI partial sums are added at the end with lane swaps.

template <int EPI>
__device__ __forceinline__ float add_parts(float v) {
  static_assert(EPI == 1 || EPI == 2 || EPI == 4 || EPI == 8, "1, 2, 4 or 8 entries per instruction");
  if constexpr (EPI >= 2) {  // lanes l and l ^ 32
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  if constexpr (EPI >= 4) {  // lanes l and l ^ 16
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  if constexpr (EPI == 8) {  // lanes l and l ^ 8 (row_ror 8 inside a 16-lane row)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  }
  return v;
}

template <Dt D>
__device__ __forceinline__ void fma16(float (&acc)[16 / DtT<D>::size], float c, const u32x4_t &w) {
  if constexpr (D == Dt::BF16) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t wv = w[v];
      acc[2 * v] = fmaf(c, bf16lo(wv), acc[2 * v]);
      acc[2 * v + 1] = fmaf(c, bf16hi(wv), acc[2 * v + 1]);
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t wv = w[v];
      acc[v] = fmaf(c, __uint_as_float(wv), acc[v]);
    }
  }
}

template <Dt D, int U>
__global__ __launch_bounds__(SP_THREADS) void k_bw_dx(RowSrc<typename DtT<D>::T> s, const f32x2_t *__restrict__ ent,
                                                     const typename DtT<D>::T *__restrict__ wu,
                                                     const typename DtT<D>::T *__restrict__ wg,
                                                     typename DtT<D>::T *__restrict__ dx, int d, int n_slices,
                                                     int tok_per_wg, int n_tb, const int *__restrict__ order) {
  using TT = typename DtT<D>::T;
  constexpr int CPL = 16 / sizeof(TT);
  constexpr int LPE = DX_SLICE / CPL;
  constexpr int EPI = 64 / LPE;
  constexpr int STEP = U * EPI;
  static_assert(STEP <= 64 && 64 % STEP == 0, "a 64-entry chunk holds whole iterations");
  __shared__ u32x4_t chunk[SP_WAVES][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int part = lane / LPE, lcol = (lane % LPE) * CPL;
  int sl, tb;
  group_coords(blockIdx.x, n_slices, n_tb, sl, tb);
  if (sl >= n_slices) return;
  const size_t w_bytes = ((size_t)s.F * d - (size_t)sl * DX_SLICE) * sizeof(TT);
  const __amdgpu_buffer_rsrc_t wur = buffer_rsrc(wu + sl * DX_SLICE, w_bytes),
                               wgr = buffer_rsrc(wg + sl * DX_SLICE, w_bytes);
  const uint32_t lane_off = lcol * sizeof(TT);
  const uint32_t row_bytes = (uint32_t)d * sizeof(TT);
  u32x4_t *C = chunk[wave];
  // the workgroup's rows, one per lane (tok_per_wg <= 64), read once
  const int r_i = min(tb * tok_per_wg + min(lane, tok_per_wg - 1), s.T - 1);
  const int my_row = order != nullptr ? order[r_i] : r_i;
  for (int it = wave; it < tok_per_wg; it += SP_WAVES) {
    const int ti = tb * tok_per_wg + it;
    if (ti >= s.T) break;
    const int t = min(max(__builtin_amdgcn_readlane(my_row, it), 0), s.T - 1);  // a valid hybrid gives a permutation
    const RowList L = row_list(s, t);
    float acc[CPL];
#pragma unroll
    for (int v = 0; v < CPL; ++v) acc[v] = 0.f;
    for (int e0 = 0; e0 < L.n; e0 += 64) {
      const int ne = min(64, L.n - e0);
      if (lane < ne) {
        const int j = clamp_col(L.col[e0 + lane], s.F);
        const f32x2_t g = ent[L.slot0 + e0 + lane];
        C[lane] = u32x4_t{(uint32_t)j * row_bytes, __float_as_uint(g[0]), __float_as_uint(g[1]), 0u};
      }
      wave_sync_lds();
      for (int e = 0; e < ne; e += STEP) {
        u32x4_t a[U], b[U];
        float cu[U], cg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = e + EPI * u + part;
          const bool ok = q < ne;
          const u32x4_t en = C[ok ? q : 0];
          cu[u] = ok ? __uint_as_float(en[1]) : 0.f;
          cg[u] = ok ? __uint_as_float(en[2]) : 0.f;
          const uint32_t ro = ok ? en[0] : NO_ROW;  // past the list: loads return zeros
          a[u] = buffer_load<u32x4_t>(wur, lane_off + ro, 0u);
          b[u] = buffer_load<u32x4_t>(wgr, lane_off + ro, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          fma16<D>(acc, cu[u], a[u]);
          fma16<D>(acc, cg[u], b[u]);
        }
      }
      wave_sync_lds();
    }
#pragma unroll
    for (int v = 0; v < CPL; ++v) acc[v] = add_parts<EPI>(acc[v]);
    u32x4_t out;
    if constexpr (D == Dt::BF16) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        out[v] = (uint32_t)bf16_rne(acc[2 * v]) | ((uint32_t)bf16_rne(acc[2 * v + 1]) << 16);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) out[v] = __float_as_uint(acc[v]);
    }
    if (part == 0) *reinterpret_cast<u32x4_t *>(dx + (size_t)t * d + sl * DX_SLICE + lcol) = out;
  }
}

// v (+ base) to p.
template <int CPL>
__device__ __forceinline__ void store_f32(float *p, const float (&v)[CPL], const f32x4_t (&base)[CPL / 4]) {
#pragma unroll
  for (int q = 0; q < CPL; q += 4)
    *reinterpret_cast<f32x4_t *>(p + q) = f32x4_t{v[q], v[q + 1], v[q + 2], v[q + 3]} + base[q / 4];
}
// The values a unit's gradient slice already holds (the dense rows' part),
// loaded when its list starts so that the loads overlap the walk; zero when
// there is nothing to add or the lane does not store.
template <int CPL>
__device__ __forceinline__ void load_base(f32x4_t (&b)[CPL / 4], const float *p, bool on) {
#pragma unroll
  for (int q = 0; q < CPL; q += 4) b[q / 4] = on ? *reinterpret_cast<const f32x4_t *>(p + q) : f32x4_t{};
}

// PART 0 forms dW_g and dW_u from the x rows, PART 1 dW_d from the dy rows.
template <Dt D, int U, int PART>
__global__ __launch_bounds__(SP_THREADS) void k_bw_dw(const int *__restrict__ colptr, const u32x4_t *__restrict__ csc,
                                                     const typename DtT<D>::T *__restrict__ x,
                                                     const typename DtT<D>::T *__restrict__ dy,
                                                     float *__restrict__ dwg, float *__restrict__ dwu,
                                                     float *__restrict__ dwd, int T, int F, int d, int n_slices,
                                                     int units_per_wg, int n_ub, const int *__restrict__ n_dense,
                                                     int dense_cap, bool dense_mma) {
  using TT = typename DtT<D>::T;
  constexpr int CPL = 16 / sizeof(TT);
  constexpr int LPE = DW_SLICE / CPL;
  constexpr int EPI = 64 / LPE;
  constexpr int STEP = U * EPI;
  static_assert(STEP <= 64 && 64 % STEP == 0, "a 64-entry chunk holds whole iterations");
  __shared__ u32x4_t chunk[SP_WAVES][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int part = lane / LPE, lcol = (lane % LPE) * CPL;
  int sl, ub;
  group_coords(blockIdx.x, n_slices, n_ub, sl, ub);
  if (sl >= n_slices) return;
  // dense rows on the matrix cores: their part of the gradients is written
  // already, and this kernel adds the other rows' sums to it
  const bool add = dense_mma && T > 0 && dense_cap > 0 && min(*n_dense, dense_cap) > 0;
  const size_t a_bytes = ((size_t)T * d - (size_t)sl * DW_SLICE) * sizeof(TT);
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x + sl * DW_SLICE, a_bytes), gr = buffer_rsrc(dy + sl * DW_SLICE, a_bytes);
  const uint32_t lane_off = lcol * sizeof(TT);
  const uint32_t row_bytes = (uint32_t)d * sizeof(TT);
  u32x4_t *C = chunk[wave];
  for (int it = wave; it < units_per_wg; it += SP_WAVES) {
    const int j = ub * units_per_wg + it;
    if (j >= F) break;
    const int c0 = colptr[j], n = colptr[j + 1] - c0;
    const size_t o = (size_t)j * d + sl * DW_SLICE + lcol;
    f32x4_t bg[CPL / 4], bu[CPL / 4], bd[CPL / 4];
    if (PART == 0) {
      load_base<CPL>(bg, dwg + o, add && part == 0);
      load_base<CPL>(bu, dwu + o, add && part == 0);
    } else {
      load_base<CPL>(bd, dwd + o, add && part == 0);
    }
    float ag[CPL], au[CPL], ad[CPL];
#pragma unroll
    for (int v = 0; v < CPL; ++v) ag[v] = au[v] = ad[v] = 0.f;
    for (int e0 = 0; e0 < n; e0 += 64) {
      const int ne = min(64, n - e0);
      if (lane < ne) {
        u32x4_t r = csc[c0 + e0 + lane];
        r[0] = min(r[0], (uint32_t)(T - 1)) * row_bytes;  // token row -> byte offset of its x / dy row
        C[lane] = r;
      }
      wave_sync_lds();
      for (int e = 0; e < ne; e += STEP) {
        u32x4_t a[U], b[U];
        float ca[U], cu[U], cg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = e + EPI * u + part;
          const bool ok = q < ne;
          const u32x4_t en = C[ok ? q : 0];
          ca[u] = ok ? __uint_as_float(en[1]) : 0.f;
          cu[u] = ok ? __uint_as_float(en[2]) : 0.f;
          cg[u] = ok ? __uint_as_float(en[3]) : 0.f;
          const uint32_t ro = ok ? en[0] : NO_ROW;  // past the list: loads return zeros
          if (PART == 0) a[u] = buffer_load<u32x4_t>(xr, lane_off + ro, 0u);
          else b[u] = buffer_load<u32x4_t>(gr, lane_off + ro, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (PART == 0) {
            fma16<D>(ag, cg[u], a[u]);
            fma16<D>(au, cu[u], a[u]);
          } else {
            fma16<D>(ad, ca[u], b[u]);
          }
        }
      }
      wave_sync_lds();
    }
#pragma unroll
    for (int v = 0; v < CPL; ++v) {
      ag[v] = add_parts<EPI>(ag[v]);
      au[v] = add_parts<EPI>(au[v]);
      ad[v] = add_parts<EPI>(ad[v]);
    }
    if (part == 0) {
      if (PART == 0) {
        store_f32<CPL>(dwg + o, ag, bg);
        store_f32<CPL>(dwu + o, au, bu);
      } else {
        store_f32<CPL>(dwd + o, ad, bd);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launch sequence.

static int bw_blocks(int T) { return (T + BW_RB - 1) / BW_RB; }

template <Dt D, int NC>
static hipError_t launch_entries(const BackwardArgs &a, const RowSrc<typename DtT<D>::T> &s, const int *order,
                                 hipStream_t st) {
  using TT = typename DtT<D>::T;
  constexpr int U = NC <= 4 ? 2 : 1;
  // hidden units per group: about 4 MB of W_u and W_d rows (one XCD's L2);
  // of W_d rows only when the forward's u is given (rows without a saved u
  // then gather from twice that)
  const size_t unit_bytes = (size_t)(a.u != nullptr ? 1 : 2) * a.d * sizeof(TT);
  int upg = (int)std::max<size_t>(64, ((size_t)4 << 20) / unit_bytes);
  upg = std::min(upg, a.F);
  const int n_groups = (a.F + upg - 1) / upg;
  const int tok = 16;
  const int n_tb = (a.T + tok - 1) / tok;
  hipLaunchKernelGGL((k_bw_entries<D, NC, U>), dim3(padded_groups(n_groups) * n_tb), dim3(SP_THREADS), 0, st, s,
                     (const TT *)a.x, (const TT *)a.dy, (const TT *)a.wu, (const TT *)a.wd, a.lam, a.d, upg,
                     n_groups, tok, n_tb, a.pos, (f32x2_t *)a.ent, (u32x4_t *)a.csc, order);
  return hipGetLastError();
}

template <Dt D>
static hipError_t launch_backward(const BackwardArgs &a, hipStream_t st) {
  using TT = typename DtT<D>::T;
  RowSrc<TT> s{a.cnt, (const TT *)a.val, a.col, a.dense_rows, a.n_dense, a.dense_cap, (const TT *)a.dense,
               a.dcol, a.dn, a.T, a.F, a.width, a.dense_mma, a.u};
  hipError_t e;
  const int NB = bw_blocks(a.T);
  const int mask_lds = a.F * 8;
  if (a.T > 0) {
    if (a.dense_cap > 0 && !a.dense_mma) {
      const int grid = std::min((a.dense_cap + BW_WAVES - 1) / BW_WAVES, 1024);
      hipLaunchKernelGGL(k_bw_dense_cols<D>, dim3(grid), dim3(BW_THREADS), 0, st, (const TT *)a.dense, a.n_dense,
                         a.dense_cap, a.F, a.dcol, a.dn);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = hipFuncSetAttribute((const void *)k_bw_count<TT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 mask_lds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(k_bw_count<TT>, dim3(NB), dim3(TR_THREADS), mask_lds, st, s, a.blk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_bw_colscan, dim3((a.F + BW_THREADS - 1) / BW_THREADS), dim3(BW_THREADS), 0, st, a.blk, NB,
                     a.F, a.boff, a.tot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the per-row kernels take the long dense rows first only when those rows
  // are walked entry by entry; with the dense rows on the matrix cores every
  // list is ELL-short and the rows go in index order (no order array)
  const int *order = a.T > 0 && !a.dense_mma ? a.order : nullptr;
  hipLaunchKernelGGL(k_bw_colptr<TT>, dim3(1), dim3(COLPTR_THREADS), 0, st, a.tot, a.F, a.colptr, s,
                     const_cast<int *>(order));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int n_slices = a.d / DX_SLICE, n_wslices = a.d / DW_SLICE;
  if (a.T > 0) {
    if ((e = hipFuncSetAttribute((const void *)k_bw_pos<TT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 mask_lds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(k_bw_pos<TT>, dim3(NB), dim3(TR_THREADS), mask_lds, st, s, a.colptr, a.boff, a.pos);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int nc = a.d / (64 * (16 / (int)sizeof(TT)));
    switch (nc) {
#define TWELL_BW_CASE(N)                                            \
  case N:                                                           \
    if ((e = launch_entries<D, N>(a, s, order, st)) != hipSuccess) return e; \
    break;
      TWELL_BW_CASE(1) TWELL_BW_CASE(2) TWELL_BW_CASE(3) TWELL_BW_CASE(4)
      TWELL_BW_CASE(5) TWELL_BW_CASE(6) TWELL_BW_CASE(7) TWELL_BW_CASE(8)
#undef TWELL_BW_CASE
      default:
        return hipErrorInvalidValue;
    }
    const int tok = 16;
    const int n_tb = (a.T + tok - 1) / tok;
    hipLaunchKernelGGL((k_bw_dx<D, 4>), dim3(padded_groups(n_slices) * n_tb), dim3(SP_THREADS), 0, st, s,
                       (const f32x2_t *)a.ent, (const TT *)a.wu, (const TT *)a.wg, (TT *)a.dx, a.d, n_slices, tok,
                       n_tb, order);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the dense rows on the matrix cores: their dx rows (after the entry
  // kernels' dx), and their part of the weight gradients (before the entry
  // kernels' weight gradients, which add onto it)
  if (a.dense_mma) {
    if ((e = ffn_backward_dense_dx(a, st)) != hipSuccess) return e;
    if ((e = ffn_backward_dense_dw(a, st)) != hipSuccess) return e;
  }
  const int upw = 8;  // units per workgroup; 8 loads in flight per lane (fastest in a sweep)
  const int n_ub = (a.F + upw - 1) / upw;
  // two passes over the transposed lists: x rows (dW_g, dW_u), then dy rows
  // (dW_d), so that each pass keeps one 256-column slice of one matrix per
  // XCD (4 MB at 8192 rows) and its loads cover two rows each
  constexpr int UDW = 8;
  hipLaunchKernelGGL((k_bw_dw<D, UDW, 0>), dim3(padded_groups(n_wslices) * n_ub), dim3(SP_THREADS), 0, st, a.colptr,
                     (const u32x4_t *)a.csc, (const TT *)a.x, (const TT *)a.dy, a.dwg, a.dwu, a.dwd, a.T, a.F, a.d,
                     n_wslices, upw, n_ub, a.n_dense, a.dense_cap, a.dense_mma);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_bw_dw<D, UDW, 1>), dim3(padded_groups(n_wslices) * n_ub), dim3(SP_THREADS), 0, st, a.colptr,
                     (const u32x4_t *)a.csc, (const TT *)a.x, (const TT *)a.dy, a.dwg, a.dwu, a.dwd, a.T, a.F, a.d,
                     n_wslices, upw, n_ub, a.n_dense, a.dense_cap, a.dense_mma);
  return hipGetLastError();
}

hipError_t ffn_backward(const BackwardArgs &a, hipStream_t s) {
  return a.dtype == Dt::BF16 ? launch_backward<Dt::BF16>(a, s) : launch_backward<Dt::F32>(a, s);
}

}  // namespace twell
