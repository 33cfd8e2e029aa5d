// Fused sparse up + down projection over TwELL entries: the single inference
// kernel of gist.science "Sparser, Faster, Lighter Transformer Language
// Models", Resumen Técnico §2.B (up and down projections in one flow from the
// TwELL gate activations, intermediate values kept in registers).
//
// One wave per token.  The wave reads the row's tile counts (a row overflows
// iff some tile counts more than cap entries: it records the flag and leaves
// the row to the dense fallback), files the row's entries in an LDS list
// (ascending unit order), holds x_t in registers and y_t as fp32 accumulators
// (d / 64 per lane, in the same lane layout as x_t), and per entry:
//   u = x_t . W_u^T[j]   (16-byte loads of the W_u row, dot2, joint reduction)
//   y_t += v W_d[j]      (v = h * u rounded to the storage dtype; 16-byte
//                         loads of the W_d row, issued with the W_u loads, FMA
//                         into the accumulators)
// so v never leaves the registers.  y_t is rounded once at the end.
// Unlike the two-kernel route, the weight rows of a token come from the whole
// of W_u and W_d, so no XCD can keep "its" rows in L2: they stream from the
// Infinity Cache / HBM.
#include "gather.hpp"
#include "launch.hpp"

#include <algorithm>

namespace twell {

constexpr int FUSED_LIST = 256;  // entries per LDS list pass (tiles per pass * cap)

// Lane of the 16-lane row holding the total of entry u after Reduce<U>.
template <int U>
__device__ __forceinline__ int reduce_lane(int u) {
  if constexpr (U == 4) return ((u & 1) << 5) | ((u >> 1) << 4);  // entries 0, 1, 2, 3 -> rows 0, 2, 1, 3
  else return u << 5;                                             // entries 0, 1 -> rows 0, 2; U = 1: lane 0
}

// GROUPED = false: one wave per token over all of the token's entries, y
// written.  GROUPED = true: hidden-group-major.  Units are cut into groups of
// tpg TwELL tiles (W_u and W_d rows of a group about one XCD's 4 MB L2, group
// g on XCD g % 8 as in the up projection); the wave of (group g, token t)
// handles t's entries in g only and writes its fp32 partial output row to
// partial[g][t][:]; k_group_reduce adds the groups' partials in group order.
// TILE_MAJOR: the TwELL records of (row t, tile k) sit at k * T + t (a tile's
// records contiguous over the tokens), else at t * nt + k; only where the
// counts and slots are read from changes.
template <Dt D, int NC, int U, bool GROUPED, bool TILE_MAJOR = false>
__global__ __launch_bounds__(SP_THREADS) void k_sparse_fused(
    const typename DtT<D>::T *__restrict__ x, const typename DtT<D>::T *__restrict__ wu,
    const typename DtT<D>::T *__restrict__ wd, const uint16_t *__restrict__ cnt,
    const typename DtT<D>::T *__restrict__ val, const uint8_t *__restrict__ idx, uint8_t *__restrict__ row_flag,
    typename DtT<D>::T *__restrict__ y, int T, int d, int nt, int tile, int cap, int tpg, int n_groups,
    int tok_per_wg, int n_tb, float *__restrict__ partial) {
  using TT = typename DtT<D>::T;
  constexpr int EPC = 16 / sizeof(TT);
  __shared__ u32x2_t lists[SP_WAVES][FUSED_LIST];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int g = 0, tb = 0;
  if constexpr (GROUPED) {
    group_coords(blockIdx.x, n_groups, n_tb, g, tb);
    if (g >= n_groups) return;
  }
  const int k_begin = GROUPED ? g * tpg : 0, k_end = GROUPED ? min(nt, (g + 1) * tpg) : nt;
  for (int it = wave; it < (GROUPED ? tok_per_wg : SP_WAVES); it += SP_WAVES) {
  const int t = GROUPED ? tb * tok_per_wg + it : blockIdx.x * SP_WAVES + wave;
  if (t >= T) return;
  auto rec = [&](int k) { return TILE_MAJOR ? (size_t)k * T + t : (size_t)t * nt + k; };
  bool over = false;
  for (int kb = 0; kb < nt; kb += 64) {
    const int k = kb + lane;
    over |= k < nt && (int)cnt[rec(k)] > cap;
  }
  const bool ovf = ballot(over) != 0;
  if (lane == 0 && g == 0) row_flag[t] = ovf ? 1 : 0;
  if (ovf) continue;

  const TT *xt = x + (size_t)t * d;
  u32x4_t xr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) xr[c] = *reinterpret_cast<const u32x4_t *>(xt + (c * 64 + lane) * EPC);
  float acc[NC][EPC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int v = 0; v < EPC; ++v) acc[c][v] = 0.f;

  const size_t w_bytes = (size_t)nt * tile * d * sizeof(TT);
  const __amdgpu_buffer_rsrc_t wur = buffer_rsrc(wu, w_bytes), wdr = buffer_rsrc(wd, w_bytes);
  const uint32_t lane_off = lane * 16;
  const uint32_t row_bytes = (uint32_t)d * sizeof(TT);
  u32x2_t *L = lists[wave];
  const int tpp = min(64, FUSED_LIST / cap);  // tiles per pass: one lane per tile
  for (int k0 = k_begin; k0 < k_end; k0 += tpp) {
    const int kn = min(tpp, k_end - k0);
    // The pass's entries into the LDS list, one lane per slot (as in the
    // two-kernel up projection): tile k0 + q holds n(q) entries.
    const int n = lane < kn ? min((int)cnt[rec(k0 + lane)], cap) : 0;
    const int incl = wave_incl_scan(n);
    const int E = __builtin_amdgcn_readlane(incl, 63);
    for (int q0 = 0; q0 < kn * cap; q0 += 64) {
      const int q = q0 + lane;
      const int kq = q / cap, sq = q - kq * cap;
      const int nq = __shfl(n, kq & 63, 64);
      const int oq = __shfl(incl - n, kq & 63, 64) + sq;
      if (q < kn * cap && sq < nq) {
        const size_t sl = rec(k0 + kq) * cap + sq;  // the slot
        const uint32_t j = (uint32_t)((k0 + kq) * tile + (idx[sl] & (tile - 1)));
        L[oq] = u32x2_t{j * row_bytes, __float_as_uint(to_f32(val[sl]))};
      }
    }
    wave_sync_lds();
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int ne = min(64, E - e0);
      const u32x2_t me = L[e0 + min(lane, ne - 1)];
      for (int u0 = 0; u0 < ne; u0 += U) {
        u32x4_t a[U][NC], b[U][NC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t off = read_lane(me[0], min(u0 + u, ne - 1));
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
        float p[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          p[u] = 0.f;
#pragma unroll
          for (int c = 0; c < NC; ++c) p[u] = dot16(xr[c], a[u][c], p[u], TT());
        }
        const float tot = Reduce<U>::run(p);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float h = __uint_as_float(read_lane(me[1], min(u0 + u, ne - 1)));
          const float uu = __uint_as_float(read_lane(__float_as_uint(tot), reduce_lane<U>(u)));
          // v = h * u rounded to the storage dtype (the down projection's input
          // activation, rounded as on every other path)
          const float v = u0 + u < ne ? to_f32(from_f32<D>(h * uu)) : 0.f;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            if constexpr (D == Dt::BF16) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint32_t wv = b[u][c][q];
                acc[c][2 * q] = fmaf(v, bf16lo(wv), acc[c][2 * q]);
                acc[c][2 * q + 1] = fmaf(v, bf16hi(wv), acc[c][2 * q + 1]);
              }
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint32_t wv = b[u][c][q];
                acc[c][q] = fmaf(v, __uint_as_float(wv), acc[c][q]);
              }
            }
          }
        }
      }
    }
    wave_sync_lds();
  }
  if constexpr (GROUPED) {
    float *pt = partial + ((size_t)g * T + t) * d;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int q = 0; q < EPC; q += 4)
        *reinterpret_cast<f32x4_t *>(pt + (c * 64 + lane) * EPC + q) =
            f32x4_t{acc[c][q], acc[c][q + 1], acc[c][q + 2], acc[c][q + 3]};
  } else {
    TT *yt = y + (size_t)t * d;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4_t out;
      if constexpr (D == Dt::BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          out[q] = (uint32_t)bf16_rne(acc[c][2 * q]) | ((uint32_t)bf16_rne(acc[c][2 * q + 1]) << 16);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = __float_as_uint(acc[c][q]);
      }
      *reinterpret_cast<u32x4_t *>(yt + (c * 64 + lane) * EPC) = out;
    }
  }
  }
}

// y of the non-overflow rows from the groups' partial rows, added in group
// order (deterministic), one rounding.  One thread per 16 bytes of y.
template <Dt D>
__global__ __launch_bounds__(256) void k_group_reduce(const float *__restrict__ partial, const uint8_t *__restrict__ row_flag,
                                                      typename DtT<D>::T *__restrict__ y, int T, int d, int n_groups) {
  using TT = typename DtT<D>::T;
  constexpr int EPC = 16 / sizeof(TT);
  const size_t chunks = (size_t)T * d / EPC;
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < chunks; q += (size_t)gridDim.x * 256) {
    const size_t e0 = q * EPC;
    const int t = (int)(e0 / d);
    if (row_flag[t] != 0) continue;  // the dense fallback writes it
    float s[EPC];
#pragma unroll
    for (int k = 0; k < EPC; ++k) s[k] = 0.f;
    for (int g = 0; g < n_groups; ++g) {
      const float *p = partial + (size_t)g * T * d + e0;
#pragma unroll
      for (int k = 0; k < EPC; k += 4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(p + k);
        s[k] += v[0];
        s[k + 1] += v[1];
        s[k + 2] += v[2];
        s[k + 3] += v[3];
      }
    }
    u32x4_t out;
    if constexpr (D == Dt::BF16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = (uint32_t)bf16_rne(s[2 * k]) | ((uint32_t)bf16_rne(s[2 * k + 1]) << 16);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = __float_as_uint(s[k]);
    }
    *reinterpret_cast<u32x4_t *>(y + e0) = out;
  }
}

template <Dt D, int NC>
static hipError_t launch_fused(const SparseArgs &a, hipStream_t s) {
  using TT = typename DtT<D>::T;
  constexpr int U = NC <= 4 ? 2 : 1;
  const int blocks = (a.T + SP_WAVES - 1) / SP_WAVES;
  hipLaunchKernelGGL((k_sparse_fused<D, NC, U, false>), dim3(blocks), dim3(SP_THREADS), 0, s, (const TT *)a.x,
                     (const TT *)a.wu, (const TT *)a.wd, a.cnt, (const TT *)a.val, a.idx, a.row_flag, (TT *)a.y, a.T,
                     a.d, a.F / a.tile, a.tile, a.cap, 0, 1, SP_WAVES, blocks, nullptr);
  return hipGetLastError();
}

template <Dt D, int NC>
static hipError_t launch_grouped(const SparseArgs &a, float *partial, hipStream_t s) {
  using TT = typename DtT<D>::T;
  constexpr int U = NC <= 4 ? 2 : 1;
  const FusedGroups fg = fused_groups(a.d, a.F, a.tile, a.dtype);
  const int tok = 16;
  const int n_tb = (a.T + tok - 1) / tok;
  auto kern = a.tile_major ? k_sparse_fused<D, NC, U, true, true> : k_sparse_fused<D, NC, U, true, false>;
  hipLaunchKernelGGL(kern, dim3(padded_groups(fg.n_groups) * n_tb), dim3(SP_THREADS), 0, s, (const TT *)a.x,
                     (const TT *)a.wu, (const TT *)a.wd, a.cnt, (const TT *)a.val, a.idx, a.row_flag, (TT *)a.y, a.T,
                     a.d, a.F / a.tile, a.tile, a.cap, fg.tpg, fg.n_groups, tok, n_tb, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t chunks = (size_t)a.T * a.d / (16 / sizeof(TT));
  const int blocks = (int)std::min<size_t>((chunks + 255) / 256, 4096);
  hipLaunchKernelGGL(k_group_reduce<D>, dim3(blocks), dim3(256), 0, s, (const float *)partial, a.row_flag, (TT *)a.y,
                     a.T, a.d, fg.n_groups);
  return hipGetLastError();
}

template <Dt D>
static hipError_t fused_dispatch(const SparseArgs &a, float *partial, hipStream_t s) {
  using TT = typename DtT<D>::T;
  const int nc = a.d / (64 * (16 / (int)sizeof(TT)));
  switch (nc) {
#define TWELL_FUSED_CASE(N) \
  case N:                   \
    return partial ? launch_grouped<D, N>(a, partial, s) : launch_fused<D, N>(a, s);
    TWELL_FUSED_CASE(1) TWELL_FUSED_CASE(2) TWELL_FUSED_CASE(3) TWELL_FUSED_CASE(4)
    TWELL_FUSED_CASE(5) TWELL_FUSED_CASE(6) TWELL_FUSED_CASE(7) TWELL_FUSED_CASE(8)
#undef TWELL_FUSED_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t sparse_fused(const SparseArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.tile_major) return hipErrorInvalidValue;  // the token-major kernel reads row-major records only
  return a.dtype == Dt::BF16 ? fused_dispatch<Dt::BF16>(a, nullptr, s) : fused_dispatch<Dt::F32>(a, nullptr, s);
}

hipError_t sparse_fused_grouped(const SparseArgs &a, float *partial, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  return a.dtype == Dt::BF16 ? fused_dispatch<Dt::BF16>(a, partial, s) : fused_dispatch<Dt::F32>(a, partial, s);
}

}  // namespace twell
